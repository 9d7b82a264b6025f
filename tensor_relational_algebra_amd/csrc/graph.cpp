// graph.cpp -- EinGraph executor.
//
// Page "EinDecomp：基于爱因斯坦求和与张量关系代数的自动张量并行分解算法":
//  * section 2.1: an EinGraph is a DAG whose nodes are EinSums and whose
//    edges are tensors (the multi-head-attention example: projections,
//    scores, softmax, weighted sum, output projection); softmax is itself
//    expressible with EinSums;
//  * section 2.2: when one node's output partitioning differs from what the
//    next node's input needs, a repartition is inserted;
//  * section 4.1: compile every node under its d into a TRA plan, partition
//    the inputs, run the plans in order and reorganise intermediates.
// On one GPU the "devices" of the pages are the workgroups of each kernel,
// and every intermediate relation lives in one caller-provided workspace.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <string>
#include <vector>

#include "graph.h"

namespace tra {

static int gfail(int code, const std::string &m)
{
    set_error(m);
    return code;
}

static int dsize(int dt) { return dt == D_BF16 ? 2 : 4; }

struct Slot {
    int node = -1;                 // producer node, or -1 for a graph input
    int leaf = -1;                 // graph-input index when node == -1
    bool repart = false;           // a copy into `buf` is needed
    std::vector<int64_t> bounds;   // tensor extents in the consumer's operand order
    std::vector<int32_t> d_from, d_to;
    size_t buf = 0;                // workspace offset of the repartitioned copy
    int dtype = D_F32;
};

struct NodeExec {
    tra_plan_t plan = nullptr;     // the node's EinSum (softmax: LSE)
    tra_plan_t plan2 = nullptr;    // softmax: exp(S - LSE)
    std::vector<int32_t> d;        // canonical order
    Slot slot[2];
    size_t out = 0, lse = 0, scratch = 0, scratch_bytes = 0;
    int64_t out_elems = 0;
    int out_dtype = D_F32;
    // attention fusion: 1 = scores / softmax node folded into a later node
    // (enqueues nothing); 2 = weighted-sum node that runs the whole chain
    int fused = 0;
    AttnDesc att{};
    Slot qkv[3];                   // Q, K, V sources, read in place
};

// An attention chain found in the graph (node indices) and its kernel descriptor.
struct AttnChain {
    int u = -1, a = -1, w = -1;    // scores, softmax, weighted sum
    AttnDesc desc{};
};

static bool is_pow2_i(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
static int log2_i(int64_t x)
{
    int r = 0;
    while ((int64_t)1 << r < x) ++r;
    return r;
}

// One label as carried by one tensor: in-block stride, key stride, block extent.
struct LabelUse {
    int64_t bs, ks, blk;
};

// Digits of one label shared by tensors blocked differently: the index's bits
// are cut at every tensor's block boundary, so that within one bit range each
// tensor's offset is linear (all in-block or all key).
static bool label_digits(int64_t ext, const std::vector<LabelUse> &uses, Pow2Group &g)
{
    if (!is_pow2_i(ext)) return false;
    std::vector<int> cuts = {0, log2_i(ext)};
    for (const LabelUse &u : uses) {
        if (!is_pow2_i(u.blk)) return false;
        cuts.push_back(log2_i(u.blk));
    }
    std::sort(cuts.begin(), cuts.end());
    cuts.erase(std::unique(cuts.begin(), cuts.end()), cuts.end());
    std::vector<SubDim> v;
    for (int i = (int)cuts.size() - 1; i >= 1; --i) {
        const int lo = cuts[i - 1], hi = cuts[i];
        SubDim sd{(uint32_t)1 << (hi - lo), {0, 0, 0}};
        for (size_t t = 0; t < uses.size(); ++t) {
            const int split = log2_i(uses[t].blk);
            sd.st[t] = lo >= split ? uses[t].ks << (lo - split) : uses[t].bs << lo;
        }
        v.push_back(sd);
    }
    return to_pow2(v, g);
}

// A tensor operand as stored: its labels (in some node's letters), the
// extents and its partition vector, both indexed by label character.
struct Stored {
    std::string lab;
    int64_t B[128];
    int32_t d[128];
    LabelUse use(char c) const
    {
        int64_t bs[kMaxRank], ks[kMaxRank];
        relation_strides(lab, B, d, bs, ks);
        const size_t p = lab.find(c);
        return {bs[p], ks[p], B[(int)c] / d[(int)c]};
    }
    int64_t elems() const
    {
        int64_t n = 1;
        for (char c : lab) n *= B[(int)c];
        return n;
    }
};

}  // namespace tra

struct tra_graph_s {
    std::vector<tra::GNode> nodes;
    std::vector<tra::NodeExec> ex;
    std::vector<std::string> leaves;
    std::vector<int64_t> leaf_elems;
    std::vector<int32_t> leaf_dtype;
    size_t ws = 0;
    int root = -1;
    int64_t cost = 0;
    int n_repart = 0;
    int n_fused = 0;
    bool overlap = false;          // copies run on a side stream (TRA_GRAPH_OVERLAP_COPIES)
    int n_copies = 0;              // input slots that need a repartition copy (graph inputs included)
    std::vector<void *> events;    // the overlapped executor's events, created on first use
    int events_device = -1;        // the device they belong to

    ~tra_graph_s()
    {
        for (auto &e : ex) {
            tra_plan_destroy(e.plan);
            tra_plan_destroy(e.plan2);
        }
        tra::events_destroy((int)events.size(), events.data());
    }
};

using namespace tra;

// Workspace layout.  Every buffer is requested with the steps (node indices in
// execution order) during which it is live: a node's output from its own
// step to its last reader's, a repartitioned copy, the logsumexp of a softmax
// node and a node's scratch for their node's step only.  Buffers whose live
// ranges overlap get disjoint byte ranges; others may share bytes, since one
// stream runs the nodes in order (section 4.1's "reorganise intermediates",
// and the memory-aware planning of the EinDecomp page's closing remarks).
// When copies run on a side stream, a copy is live from its producer's step
// (step 0 for a graph input), when it may start, to its consumer's.
struct WsReq {
    size_t *at;        // where the assigned offset is written
    size_t bytes;
    int first, last;   // live steps, inclusive
};

static void request(std::vector<WsReq> &reqs, size_t *at, size_t bytes, int first, int last = -1)
{
    reqs.push_back({at, bytes, first, last < 0 ? first : last});
}

// First fit in a given order; returns the extent and the offsets.
static size_t first_fit(const std::vector<WsReq> &reqs, const std::vector<size_t> &order, std::vector<size_t> &at_out)
{
    at_out.assign(reqs.size(), 0);
    struct Placed {
        size_t lo, hi;
        int first, last;
    };
    std::vector<Placed> placed;
    size_t extent = 0;
    for (size_t i : order) {
        const WsReq &r = reqs[i];
        const size_t need = (r.bytes + 255) & ~(size_t)255;
        std::vector<std::pair<size_t, size_t>> busy;
        for (const Placed &p : placed)
            if (p.first <= r.last && r.first <= p.last) busy.push_back({p.lo, p.hi});
        std::sort(busy.begin(), busy.end());
        size_t at = 0;
        for (auto &b : busy) {
            if (at + need <= b.first) break;
            at = std::max(at, b.second);
        }
        at_out[i] = at;
        placed.push_back({at, at + need, r.first, r.last});
        extent = std::max(extent, at + need);
    }
    return extent;
}

// Two first-fit layouts, largest buffer first (the large long-lived tensors
// leave holes the small ones fill) and in order of first use; the smaller
// extent is kept and its offsets written.  Returns the extent.
static size_t assign_offsets(std::vector<WsReq> &reqs)
{
    std::vector<size_t> by_size(reqs.size()), by_use(reqs.size());
    for (size_t i = 0; i < reqs.size(); ++i) by_size[i] = by_use[i] = i;
    std::stable_sort(by_size.begin(), by_size.end(), [&](size_t a, size_t b) {
        if (reqs[a].bytes != reqs[b].bytes) return reqs[a].bytes > reqs[b].bytes;
        return reqs[a].first < reqs[b].first;
    });
    std::stable_sort(by_use.begin(), by_use.end(), [&](size_t a, size_t b) {
        if (reqs[a].first != reqs[b].first) return reqs[a].first < reqs[b].first;
        return reqs[a].bytes > reqs[b].bytes;
    });
    std::vector<size_t> at_a, at_b;
    const size_t ea = first_fit(reqs, by_size, at_a), eb = first_fit(reqs, by_use, at_b);
    const std::vector<size_t> &at = ea <= eb ? at_a : at_b;
    for (size_t i = 0; i < reqs.size(); ++i) *reqs[i].at = at[i];
    return std::min(ea, eb);
}

// Resolve node v's input slot s to its producer output or graph input, with
// no repartition (the fused kernel reads every operand in its stored blocking).
static int source_slot(tra_graph_s *g, int v, int s, Slot &sl)
{
    const GNode &nd = g->nodes[v];
    sl = Slot{};
    sl.dtype = nd.in_dtype;
    int64_t elems = 1;
    for (char c : nd.ops[s]) elems *= nd.B[(int)c];
    if (nd.src[s] >= 0) {
        sl.node = nd.src[s];
        return TRA_OK;
    }
    const std::string name = nd.inputs[s].substr(1);
    int li = -1;
    for (size_t i = 0; i < g->leaves.size(); ++i)
        if (g->leaves[i] == name) li = (int)i;
    if (li < 0) {
        li = (int)g->leaves.size();
        g->leaves.push_back(name);
        g->leaf_elems.push_back(elems);
        g->leaf_dtype.push_back(nd.in_dtype);
    } else if (g->leaf_elems[li] != elems || g->leaf_dtype[li] != nd.in_dtype) {
        return gfail(TRA_E_GRAPH, "graph input @" + name + " is used with two shapes or dtypes");
    }
    sl.leaf = li;
    return TRA_OK;
}

// The weighted-sum node of a fused chain: sources of Q, K (the scores node's
// inputs) and V, and the node's output buffer in its own blocking.
static int plan_fused(tra_graph_s *g, int w, std::vector<WsReq> &reqs, std::vector<int> &out_req)
{
    NodeExec &e = g->ex[w];
    const GNode &W = g->nodes[w];
    const int a = W.src[0], u = g->nodes[a].src[0];
    int rc = source_slot(g, u, 0, e.qkv[0]);
    if (!rc) rc = source_slot(g, u, 1, e.qkv[1]);
    if (!rc) rc = source_slot(g, w, 1, e.qkv[2]);
    if (rc) return rc;
    e.out_dtype = W.out_dtype;
    e.out_elems = 1;
    for (char c : W.out) e.out_elems *= W.B[(int)c];
    out_req[w] = (int)reqs.size();
    request(reqs, &e.out, (size_t)e.out_elems * dsize(W.out_dtype), w, w);
    return TRA_OK;
}

// The stored form of node v's input slot s (its producer's blocking, or dense
// for a graph input), in node v's letters.
static Stored stored_input(const std::vector<GNode> &nodes, const std::vector<std::vector<int32_t>> &ds, int v, int s)
{
    const GNode &nd = nodes[v];
    Stored t;
    t.lab = nd.ops[s];
    for (int i = 0; i < 128; ++i) {
        t.B[i] = nd.B[i];
        t.d[i] = 1;
    }
    const int u = nd.src[s];
    if (u >= 0)
        for (size_t i = 0; i < t.lab.size(); ++i) t.d[(int)t.lab[i]] = ds[u][nodes[u].canon.find(nodes[u].out[i])];
    return t;
}

// Find every scores -> softmax -> weighted-sum chain the fused kernel can run
// and build its descriptor; chains that do not fit are left to the unfused path.
static std::vector<AttnChain> find_attention(const std::vector<GNode> &nodes,
                                             const std::vector<std::vector<int32_t>> &ds, const std::vector<int> &uses)
{
    std::vector<AttnChain> out;
    const int n = (int)nodes.size();
    for (int a = 0; a < n; ++a) {
        const GNode &A = nodes[a];
        if (A.kind != "softmax" || A.src.size() != 1 || A.src[0] < 0) continue;
        const int u = A.src[0];
        const GNode &U = nodes[u];
        if (U.kind != "einsum" || U.ops.size() != 2 || uses[u] != 1 || uses[a] != 1) continue;
        int w = -1;
        for (int x = 0; x < n; ++x)
            for (int sidx : nodes[x].src)
                if (sidx == a) w = x;
        if (w < 0) continue;
        const GNode &W = nodes[w];
        if (W.kind != "einsum" || W.ops.size() != 2 || W.src[0] != a || W.src[1] == a) continue;
        // roles in the scores node: S[h, s, t] from Q[s, h, d] and K[t, h, d]
        const std::string &Q = U.ops[0], &K = U.ops[1], &S = U.out;
        if (S.size() != 3 || Q.size() != 3 || K.size() != 3 || U.con.size() != 1) continue;
        char h = 0, sq = 0, tk = 0;
        for (char c : S) {
            const bool inq = Q.find(c) != std::string::npos, ink = K.find(c) != std::string::npos;
            if (inq && ink) h = c;
            else if (inq) sq = c;
            else if (ink) tk = c;
        }
        const char dq = U.con[0];
        if (!h || !sq || !tk || S.back() != tk) continue;
        // the weighted-sum node in its own letters: A positionally matches S
        const std::string &Al = W.ops[0], &Vl = W.ops[1], &Ol = W.out;
        if (Al.size() != 3 || Vl.size() != 3 || Ol.size() != 3 || W.con.size() != 1) continue;
        const char hw = Al[S.find(h)], sw = Al[S.find(sq)], tw = Al[S.find(tk)];
        if (W.con[0] != tw) continue;
        char dv = 0;
        for (char c : Vl)
            if (c != tw && c != hw) dv = c;
        if (!dv || Vl.find(tw) == std::string::npos || Vl.find(hw) == std::string::npos) continue;
        if (Ol.find(sw) == std::string::npos || Ol.find(hw) == std::string::npos || Ol.find(dv) == std::string::npos)
            continue;
        const int64_t Sx = U.B[(int)sq], Tx = U.B[(int)tk], Hx = U.B[(int)h], Dx = U.B[(int)dq];
        if (W.B[(int)sw] != Sx || W.B[(int)tw] != Tx || W.B[(int)hw] != Hx || W.B[(int)dv] != Dx) continue;
        if (U.in_dtype != D_BF16 || W.in_dtype != D_BF16 || W.scale != 1.0f) continue;
        if ((Dx != 32 && Dx != 64 && Dx != 128) || Sx % 128 || Tx % 64) continue;

        const Stored sQ = stored_input(nodes, ds, u, 0), sK = stored_input(nodes, ds, u, 1);
        const Stored sV = stored_input(nodes, ds, w, 1);
        Stored sO;
        sO.lab = Ol;
        for (int i = 0; i < 128; ++i) {
            sO.B[i] = W.B[i];
            sO.d[i] = 1;
        }
        for (size_t i = 0; i < W.canon.size(); ++i) sO.d[(int)W.canon[i]] = ds[w][i];

        AttnChain ch;
        ch.u = u;
        ch.a = a;
        ch.w = w;
        AttnDesc &ad = ch.desc;
        bool ok = label_digits(Sx, {sQ.use(sq), sO.use(sw)}, ad.gs) &&
                  label_digits(Tx, {sK.use(tk), sV.use(tw)}, ad.gt) &&
                  label_digits(Hx, {sQ.use(h), sK.use(h), sV.use(hw)}, ad.gh) &&
                  label_digits(Hx, {sO.use(hw)}, ad.gho) &&
                  label_digits(Dx, {sQ.use(dq), sK.use(dq), sV.use(dv)}, ad.gd) &&
                  label_digits(Dx, {sO.use(dv)}, ad.gdo);
        if (!ok) continue;
        // Q, K, V are read in 16-byte runs along the head dimension
        const int ld = ad.gd.n - 1;
        if (ld < 0 || ad.gd.mask[ld] + 1 < 8 || ad.gd.st[0][ld] != 1 || ad.gd.st[1][ld] != 1 || ad.gd.st[2][ld] != 1)
            continue;
        const int lo = ad.gdo.n - 1;
        ad.o_vec4 = lo >= 0 && ad.gdo.mask[lo] + 1 >= 4 && ad.gdo.st[0][lo] == 1;
        if (sQ.elems() >= (1ll << 31) || sK.elems() >= (1ll << 31) || sV.elems() >= (1ll << 31) ||
            sO.elems() >= (1ll << 31))
            continue;
        // the largest offset the kernel can form in each tensor stays inside it
        auto reach = [](const Pow2Group &g, int t) {
            int64_t m = 0;
            for (int i = 0; i < g.n; ++i) m += (int64_t)g.mask[i] * g.st[t][i];
            return m;
        };
        if (reach(ad.gs, 0) + reach(ad.gh, 0) + reach(ad.gd, 0) >= sQ.elems() ||
            reach(ad.gt, 0) + reach(ad.gh, 1) + reach(ad.gd, 1) >= sK.elems() ||
            reach(ad.gt, 1) + reach(ad.gh, 2) + reach(ad.gd, 2) >= sV.elems() ||
            reach(ad.gs, 1) + reach(ad.gho, 0) + reach(ad.gdo, 0) >= sO.elems())
            continue;   // never true for a valid relation layout
        ad.S = (uint32_t)Sx;
        ad.T = (uint32_t)Tx;
        ad.H = (uint32_t)Hx;
        ad.D = (uint32_t)Dx;
        ad.scale_log2 = U.scale * 1.4426950408889634f;
        out.push_back(ch);
    }
    return out;
}

static int graph_plan(const char *graph_desc, int P, const int32_t *d_all, int d_len, int flags, int64_t mem_cap,
                      tra_graph_t *out);

extern "C" int tra_graph_plan(const char *graph_desc, int P, const int32_t *d_all, int d_len, tra_graph_t *out)
{
    return graph_plan(graph_desc, P, d_all, d_len, 0, 0, out);
}

extern "C" int tra_graph_plan_ex(const char *graph_desc, int P, const int32_t *d_all, int d_len, int flags,
                                 tra_graph_t *out)
{
    return graph_plan(graph_desc, P, d_all, d_len, flags, 0, out);
}

extern "C" int tra_graph_plan_cap(const char *graph_desc, int P, int flags, int64_t mem_cap_bytes, tra_graph_t *out)
{
    if (mem_cap_bytes < 0) return gfail(TRA_E_OP, "negative memory cap");
    return graph_plan(graph_desc, P, nullptr, 0, flags, mem_cap_bytes, out);
}

static int graph_plan(const char *graph_desc, int P, const int32_t *d_all, int d_len, int flags, int64_t mem_cap,
                      tra_graph_t *out)
{
    if (!graph_desc || !out) return gfail(TRA_E_NULL, "graph_desc / out is NULL");
    if (flags & ~(TRA_GRAPH_FUSE_ATTENTION | TRA_GRAPH_CHOOSE_TIME | TRA_GRAPH_OVERLAP_COPIES))
        return gfail(TRA_E_OP, "unknown graph flag");
    *out = nullptr;
    tra_graph_s *g = new tra_graph_s();
    g->overlap = (flags & TRA_GRAPH_OVERLAP_COPIES) != 0;
    auto bad = [&](int rc) {
        delete g;
        return rc;
    };
    int rc = parse_graph(graph_desc, g->nodes);
    if (rc) return bad(rc);
    const size_t n = g->nodes.size();
    std::vector<std::vector<int32_t>> ds;
    if (d_all) {
        size_t pos = 0;
        for (auto &nd : g->nodes) {
            if (pos + nd.canon.size() > (size_t)d_len) return bad(gfail(TRA_E_DLEN, "d_all too short"));
            ds.emplace_back(d_all + pos, d_all + pos + nd.canon.size());
            pos += nd.canon.size();
        }
        if (pos != (size_t)d_len) return bad(gfail(TRA_E_DLEN, "d_all has extra entries"));
        g->cost = -1;
    } else {
        rc = run_dp(g->nodes, P, ds, g->cost, (flags & TRA_GRAPH_CHOOSE_TIME) ? COST_TIME : COST_PAGES, mem_cap);
        if (rc) return bad(rc);
    }
    std::vector<int> uses(n, 0);
    for (auto &nd : g->nodes)
        for (int s : nd.src)
            if (s >= 0) uses[s]++;
    for (size_t v = 0; v < n; ++v)
        if (!uses[v]) g->root = (int)v;

    g->ex.resize(n);
    if (flags & TRA_GRAPH_FUSE_ATTENTION) {
        for (const AttnChain &ch : find_attention(g->nodes, ds, uses)) {
            g->ex[ch.u].fused = 1;
            g->ex[ch.a].fused = 1;
            g->ex[ch.w].fused = 2;
            g->ex[ch.w].att = ch.desc;
            g->n_fused++;
        }
    }
    std::vector<WsReq> reqs;
    std::vector<int> out_req(n, -1);   // index of each node's output request
    for (size_t v = 0; v < n; ++v) {
        GNode &nd = g->nodes[v];
        NodeExec &e = g->ex[v];
        e.d = ds[v];
        if (e.fused == 1) continue;   // folded into its weighted-sum node
        if (e.fused == 2) {
            rc = plan_fused(g, (int)v, reqs, out_req);
            if (rc) return bad(rc);
            continue;
        }
        std::vector<int64_t> bounds;
        for (char c : nd.canon) bounds.push_back(nd.B[(int)c]);
        int32_t dmap[128];
        for (int i = 0; i < 128; ++i) dmap[i] = 1;
        for (size_t i = 0; i < nd.canon.size(); ++i) dmap[(int)nd.canon[i]] = e.d[i];
        e.out_dtype = nd.out_dtype;
        if (nd.kind == "softmax") {
            if (nd.in_dtype != D_F32) return bad(gfail(TRA_E_GRAPH, "a softmax node reads fp32 scores (in=f32)"));
            const std::string hst = nd.out, hs = nd.out.substr(0, nd.out.size() - 1);
            rc = tra_plan((hst + "->" + hs).c_str(), bounds.data(), e.d.data(), (int)bounds.size(), TRA_JOIN_IDENT,
                          TRA_AGG_LSE, nd.in_dtype, D_F32, 1.0f, &e.plan);
            if (rc) return bad(rc);
            rc = tra_plan((hst + "," + hs + "->" + hst).c_str(), bounds.data(), e.d.data(), (int)bounds.size(),
                          TRA_JOIN_EXP_SUB, TRA_AGG_NONE, nd.in_dtype, nd.out_dtype, 1.0f, &e.plan2);
            if (rc) return bad(rc);
        } else {
            rc = tra_plan(nd.spec.c_str(), bounds.data(), e.d.data(), (int)bounds.size(), TRA_JOIN_MUL, TRA_AGG_SUM,
                          nd.in_dtype, nd.out_dtype, nd.scale, &e.plan);
            if (rc) return bad(rc);
        }
        tra_plan_info_t pi{};
        tra_plan_info(e.plan2 ? e.plan2 : e.plan, &pi);
        e.out_elems = pi.z_elems;
        // input slots
        for (size_t s = 0; s < nd.ops.size(); ++s) {
            Slot &sl = e.slot[s];
            const std::string &lab = nd.ops[s];
            sl.dtype = nd.in_dtype;
            for (char c : lab) {
                sl.bounds.push_back(nd.B[(int)c]);
                sl.d_to.push_back(dmap[(int)c]);
            }
            int64_t elems = 1;
            for (int64_t b : sl.bounds) elems *= b;
            if (nd.src[s] < 0) {
                std::string name = nd.inputs[s].substr(1);
                int li = -1;
                for (size_t i = 0; i < g->leaves.size(); ++i)
                    if (g->leaves[i] == name) li = (int)i;
                if (li < 0) {
                    li = (int)g->leaves.size();
                    g->leaves.push_back(name);
                    g->leaf_elems.push_back(elems);
                    g->leaf_dtype.push_back(nd.in_dtype);
                } else if (g->leaf_elems[li] != elems || g->leaf_dtype[li] != nd.in_dtype) {
                    return bad(gfail(TRA_E_GRAPH, "graph input @" + name + " is used with two shapes or dtypes"));
                }
                sl.leaf = li;
                sl.d_from.assign(lab.size(), 1);
            } else {
                const int u = nd.src[s];
                const GNode &pu = g->nodes[u];
                if (pu.out_dtype != nd.in_dtype)
                    return bad(gfail(TRA_E_GRAPH, "node " + nd.name + " reads " + pu.name + " in another dtype"));
                sl.node = u;
                for (char c : pu.out) sl.d_from.push_back(g->ex[u].d[pu.canon.find(c)]);
                if (sl.d_from != sl.d_to) g->n_repart++;
            }
            sl.repart = sl.d_from != sl.d_to;
            if (sl.repart) {
                g->n_copies++;
                request(reqs, &sl.buf, (size_t)elems * dsize(nd.in_dtype),
                        g->overlap ? std::max(sl.node, 0) : (int)v, (int)v);
            }
        }
        out_req[v] = (int)reqs.size();
        request(reqs, &e.out, (size_t)e.out_elems * dsize(nd.out_dtype), (int)v, (int)v);
        if (e.plan2) {
            tra_plan_info_t li{};
            tra_plan_info(e.plan, &li);
            request(reqs, &e.lse, (size_t)li.z_elems * 4, (int)v);
        }
        tra_plan_info(e.plan, &pi);
        size_t sb = pi.workspace_bytes;
        if (e.plan2) {
            tra_plan_info_t p2{};
            tra_plan_info(e.plan2, &p2);
            sb = std::max(sb, p2.workspace_bytes);
        }
        e.scratch_bytes = sb;
        if (sb) request(reqs, &e.scratch, sb, (int)v);
    }
    // an output stays live until its last reader's step (the root's until its
    // own step, which writes it back dense)
    for (size_t x = 0; x < n; ++x) {
        const NodeExec &e = g->ex[x];
        if (e.fused == 1) continue;
        auto reads = [&](int p) {
            if (p >= 0 && out_req[p] >= 0) reqs[out_req[p]].last = std::max(reqs[out_req[p]].last, (int)x);
        };
        if (e.fused == 2) {
            for (const Slot &sl : e.qkv) reads(sl.node);
        } else {
            for (size_t s = 0; s < g->nodes[x].ops.size(); ++s) reads(e.slot[s].node);
        }
    }
    g->ws = assign_offsets(reqs);
    if (mem_cap > 0 && (int64_t)g->ws > mem_cap)
        return bad(gfail(TRA_E_NO_CANDIDATE, "the chosen plan's workspace layout needs " + std::to_string(g->ws) +
                                                 " bytes, over the memory cap (layout fragmentation)"));
    *out = g;
    return TRA_OK;
}

extern "C" int tra_graph_info(tra_graph_t g, tra_graph_info_t *info)
{
    if (!g || !info) return gfail(TRA_E_NULL, "graph / info is NULL");
    info->n_nodes = (int32_t)g->nodes.size();
    info->n_leaves = (int32_t)g->leaves.size();
    info->workspace_bytes = g->ws;
    info->out_elems = g->ex[g->root].out_elems;
    info->out_dtype = g->ex[g->root].out_dtype;
    info->cost = g->cost;
    info->n_repartitions = g->n_repart;
    info->n_fused = g->n_fused;
    return TRA_OK;
}

extern "C" int tra_graph_node_d(tra_graph_t g, int node, int32_t *d_out, int cap)
{
    if (!g || !d_out) return gfail(TRA_E_NULL, "graph / d_out is NULL");
    if (node < 0 || node >= (int)g->nodes.size()) return gfail(TRA_E_GRAPH, "node index out of range");
    const auto &d = g->ex[node].d;
    if ((int)d.size() > cap) return gfail(TRA_E_BUFFER, "d_out too small");
    for (size_t i = 0; i < d.size(); ++i) d_out[i] = d[i];
    return (int)d.size();
}

extern "C" int tra_graph_node_output(tra_graph_t g, int node, size_t *offset, int64_t *elems, int32_t *dtype,
                                     size_t *lse_offset, int64_t *lse_elems)
{
    if (!g || !offset || !elems || !dtype || !lse_offset || !lse_elems) return gfail(TRA_E_NULL, "NULL argument");
    if (node < 0 || node >= (int)g->nodes.size()) return gfail(TRA_E_GRAPH, "node index out of range");
    const NodeExec &e = g->ex[node];
    if (e.fused == 1) return gfail(TRA_E_OP, "node is folded into a fused attention chain");
    *offset = e.out;
    *elems = e.out_elems;
    *dtype = e.out_dtype;
    const GNode &nd = g->nodes[node];
    const bool sm = nd.kind == "softmax";
    *lse_offset = sm ? e.lse : SIZE_MAX;
    *lse_elems = sm ? e.out_elems / nd.B[(int)nd.out.back()] : 0;
    return TRA_OK;
}

extern "C" int tra_graph_leaf(tra_graph_t g, int leaf, char *name, int cap, int64_t *elems, int32_t *dtype)
{
    if (!g || !name || !elems || !dtype) return gfail(TRA_E_NULL, "NULL argument");
    if (leaf < 0 || leaf >= (int)g->leaves.size()) return gfail(TRA_E_GRAPH, "leaf index out of range");
    if ((int)g->leaves[leaf].size() + 1 > cap) return gfail(TRA_E_BUFFER, "name buffer too small");
    std::memcpy(name, g->leaves[leaf].c_str(), g->leaves[leaf].size() + 1);
    *elems = g->leaf_elems[leaf];
    *dtype = g->leaf_dtype[leaf];
    return TRA_OK;
}

// The output node's relation, written dense row-major to `out`.
static int write_root(tra_graph_t g, int node, void *out, char *ws, void *stream)
{
    const NodeExec &e = g->ex[node];
    const GNode &nd = g->nodes[node];
    std::vector<int64_t> b;
    std::vector<int32_t> dz, ones;
    for (char c : nd.out) {
        b.push_back(nd.B[(int)c]);
        dz.push_back(e.d[nd.canon.find(c)]);
        ones.push_back(1);
    }
    return tra_repartition(b.data(), (int)b.size(), dz.data(), ones.data(), e.out_dtype, ws + e.out, out, stream);
}

static int check_run_args(tra_graph_t g, const void *const *leaves, int n_leaves, void *workspace, size_t ws_bytes)
{
    if (!g) return gfail(TRA_E_NULL, "graph is NULL");
    if (g->ws && (!workspace || ws_bytes < g->ws))
        return gfail(TRA_E_WORKSPACE, "graph workspace of " + std::to_string(g->ws) + " bytes needed");
    if (n_leaves != (int)g->leaves.size() || (n_leaves && !leaves))
        return gfail(TRA_E_NULL, "expected " + std::to_string(g->leaves.size()) + " graph inputs");
    return TRA_OK;
}

// The repartition of one input slot into its workspace copy.
static int run_copy(tra_graph_t g, const Slot &sl, const void *const *leaves, char *ws, void *stream)
{
    const void *src = sl.node >= 0 ? (const void *)(ws + g->ex[sl.node].out) : leaves[sl.leaf];
    if (!src) return gfail(TRA_E_NULL, "graph input pointer is NULL");
    return tra_repartition(sl.bounds.data(), (int)sl.bounds.size(), sl.d_from.data(), sl.d_to.data(), sl.dtype, src,
                           ws + sl.buf, stream);
}

// One node on `stream`; its input copies too unless copies_done (the
// overlapped executor has run them on its side stream).
static int run_node(tra_graph_t g, int node, const void *const *leaves, void *out, char *ws, void *stream,
                    bool copies_done)
{
    NodeExec &e = g->ex[node];
    const GNode &nd = g->nodes[node];
    if (e.fused == 1) return TRA_OK;   // runs inside its chain's weighted-sum node
    int rc;
    if (e.fused == 2) {
        const void *p[3];
        for (int i = 0; i < 3; ++i) {
            const Slot &sl = e.qkv[i];
            p[i] = sl.node >= 0 ? (const void *)(ws + g->ex[sl.node].out) : leaves[sl.leaf];
            if (!p[i]) return gfail(TRA_E_NULL, "graph input pointer is NULL");
        }
        rc = launch_attention(e.att, e.out_dtype, p[0], p[1], p[2], ws + e.out, stream);
        if (rc) return gfail(TRA_E_HIP, std::string("fused attention launch: ") + hip_error_text(rc));
        return node == g->root ? write_root(g, node, out, ws, stream) : TRA_OK;
    }
    const void *in[2] = {nullptr, nullptr};
    for (size_t s = 0; s < nd.ops.size(); ++s) {
        const Slot &sl = e.slot[s];
        if (sl.repart) {
            if (!copies_done) {
                rc = run_copy(g, sl, leaves, ws, stream);
                if (rc) return rc;
            }
            in[s] = ws + sl.buf;
        } else {
            in[s] = sl.node >= 0 ? (const void *)(ws + g->ex[sl.node].out) : leaves[sl.leaf];
            if (!in[s]) return gfail(TRA_E_NULL, "graph input pointer is NULL");
        }
    }
    void *scratch = e.scratch_bytes ? ws + e.scratch : nullptr;
    if (e.plan2 && softmax_one_pass(*e.plan, *e.plan2)) {
        if (!in[0]) return gfail(TRA_E_NULL, "softmax input is NULL");
        rc = launch_softmax_rows(*e.plan, *e.plan2, in[0], ws + e.lse, ws + e.out, stream);
        if (rc) return gfail(TRA_E_HIP, std::string("softmax launch: ") + hip_error_text(rc));
    } else if (e.plan2) {
        rc = tra_execute(e.plan, in[0], nullptr, ws + e.lse, scratch, e.scratch_bytes, stream);
        if (rc) return rc;
        rc = tra_execute(e.plan2, in[0], ws + e.lse, ws + e.out, scratch, e.scratch_bytes, stream);
    } else {
        rc = tra_execute(e.plan, in[0], in[1], ws + e.out, scratch, e.scratch_bytes, stream);
    }
    if (rc) return rc;
    return node == g->root ? write_root(g, node, out, ws, stream) : TRA_OK;
}

extern "C" int tra_graph_run_node(tra_graph_t g, int node, const void *const *leaves, int n_leaves, void *out,
                                  void *workspace, size_t ws_bytes, void *stream)
{
    int rc = check_run_args(g, leaves, n_leaves, workspace, ws_bytes);
    if (rc) return rc;
    if (node < 0 || node >= (int)g->nodes.size()) return gfail(TRA_E_GRAPH, "node index out of range");
    if (node == g->root && !out) return gfail(TRA_E_NULL, "the output node needs `out`");
    return run_node(g, node, leaves, out, (char *)workspace, stream, false);
}

static int hip_fail(int rc, const char *what)
{
    return gfail(TRA_E_HIP, std::string(what) + ": " + hip_error_text(rc));
}

// Nodes in order on `stream`; every repartition copy on the device's side
// stream, started as soon as its source exists (graph inputs at once, an
// intermediate when its producer has run), the consumer waiting for it.
// Events: [0] start, [1 + v] node v done, [1 + n + 2v + s] copy of v's slot s.
static int execute_overlapped(tra_graph_t g, const void *const *leaves, void *out, char *ws, void *stream)
{
    const int n = (int)g->nodes.size();
    int dev = 0, rc = current_device(&dev);
    if (rc) return hip_fail(rc, "hipGetDevice");
    void *side = nullptr;
    rc = side_stream(&side);
    if (rc) return hip_fail(rc, "side stream");
    if (g->events.empty() || g->events_device != dev) {
        events_destroy((int)g->events.size(), g->events.data());
        g->events.assign(1 + 3 * (size_t)n, nullptr);
        rc = events_create((int)g->events.size(), g->events.data());
        if (rc) {
            g->events.clear();
            return hip_fail(rc, "hipEventCreate");
        }
        g->events_device = dev;
    }
    void **ev = g->events.data();
    auto ev_node = [&](int v) { return ev[1 + v]; };
    auto ev_copy = [&](int v, int s) { return ev[1 + n + 2 * v + s]; };
    auto copy_on_side = [&](int v, int s) -> int {
        int r = run_copy(g, g->ex[v].slot[s], leaves, ws, side);
        if (r) return r;
        r = event_record(ev_copy(v, s), side);
        return r ? hip_fail(r, "hipEventRecord") : TRA_OK;
    };
    auto copies_of = [&](int v) {   // (slot count) of a node that reads through copies
        return g->ex[v].fused == 0 ? (int)g->nodes[v].ops.size() : 0;
    };
    if ((rc = event_record(ev[0], stream)) || (rc = stream_wait_event(side, ev[0])))
        return hip_fail(rc, "stream fork");
    for (int v = 0; v < n; ++v)
        for (int s = 0; s < copies_of(v); ++s)
            if (g->ex[v].slot[s].repart && g->ex[v].slot[s].node < 0 && (rc = copy_on_side(v, s))) return rc;
    for (int v = 0; v < n; ++v) {
        for (int s = 0; s < copies_of(v); ++s)
            if (g->ex[v].slot[s].repart && (rc = stream_wait_event(stream, ev_copy(v, s))))
                return hip_fail(rc, "hipStreamWaitEvent");
        rc = run_node(g, v, leaves, v == g->root ? out : nullptr, ws, stream, true);
        if (rc) return rc;
        bool forked = false;
        for (int w = v + 1; w < n; ++w)
            for (int s = 0; s < copies_of(w); ++s) {
                const Slot &sl = g->ex[w].slot[s];
                if (!sl.repart || sl.node != v) continue;
                if (!forked) {
                    if ((rc = event_record(ev_node(v), stream)) || (rc = stream_wait_event(side, ev_node(v))))
                        return hip_fail(rc, "stream fork");
                    forked = true;
                }
                if ((rc = copy_on_side(w, s))) return rc;
            }
    }
    return TRA_OK;
}

extern "C" int tra_graph_execute(tra_graph_t g, const void *const *leaves, int n_leaves, void *out, void *workspace,
                                 size_t ws_bytes, void *stream)
{
    int rc = check_run_args(g, leaves, n_leaves, workspace, ws_bytes);
    if (rc) return rc;
    if (!out) return gfail(TRA_E_NULL, "the output node needs `out`");
    if (g->overlap && g->n_copies > 0) return execute_overlapped(g, leaves, out, (char *)workspace, stream);
    for (int v = 0; v < (int)g->nodes.size(); ++v) {
        rc = run_node(g, v, leaves, v == g->root ? out : nullptr, (char *)workspace, stream, false);
        if (rc) return rc;
    }
    return TRA_OK;
}

extern "C" int tra_graph_destroy(tra_graph_t g)
{
    delete g;
    return TRA_OK;
}
