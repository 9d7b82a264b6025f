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

    ~tra_graph_s()
    {
        for (auto &e : ex) {
            tra_plan_destroy(e.plan);
            tra_plan_destroy(e.plan2);
        }
    }
};

using namespace tra;

static size_t bump(size_t &top, size_t bytes)
{
    size_t at = (top + 255) & ~(size_t)255;
    top = at + bytes;
    return at;
}

extern "C" int tra_graph_plan(const char *graph_desc, int P, const int32_t *d_all, int d_len, tra_graph_t *out)
{
    if (!graph_desc || !out) return gfail(TRA_E_NULL, "graph_desc / out is NULL");
    *out = nullptr;
    tra_graph_s *g = new tra_graph_s();
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
        rc = run_dp(g->nodes, P, ds, g->cost);
        if (rc) return bad(rc);
    }
    std::vector<int> uses(n, 0);
    for (auto &nd : g->nodes)
        for (int s : nd.src)
            if (s >= 0) uses[s]++;
    for (size_t v = 0; v < n; ++v)
        if (!uses[v]) g->root = (int)v;

    g->ex.resize(n);
    size_t top = 0;
    for (size_t v = 0; v < n; ++v) {
        GNode &nd = g->nodes[v];
        NodeExec &e = g->ex[v];
        e.d = ds[v];
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
            if (sl.repart) sl.buf = bump(top, (size_t)elems * dsize(nd.in_dtype));
        }
        e.out = bump(top, (size_t)e.out_elems * dsize(nd.out_dtype));
        if (e.plan2) {
            tra_plan_info_t li{};
            tra_plan_info(e.plan, &li);
            e.lse = bump(top, (size_t)li.z_elems * 4);
        }
        tra_plan_info(e.plan, &pi);
        size_t sb = pi.workspace_bytes;
        if (e.plan2) {
            tra_plan_info_t p2{};
            tra_plan_info(e.plan2, &p2);
            sb = std::max(sb, p2.workspace_bytes);
        }
        e.scratch_bytes = sb;
        if (sb) e.scratch = bump(top, sb);
    }
    g->ws = (top + 255) & ~(size_t)255;
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

extern "C" int tra_graph_run_node(tra_graph_t g, int node, const void *const *leaves, int n_leaves, void *out,
                                  void *workspace, size_t ws_bytes, void *stream)
{
    if (!g) return gfail(TRA_E_NULL, "graph is NULL");
    if (node < 0 || node >= (int)g->nodes.size()) return gfail(TRA_E_GRAPH, "node index out of range");
    if (g->ws && (!workspace || ws_bytes < g->ws))
        return gfail(TRA_E_WORKSPACE, "graph workspace of " + std::to_string(g->ws) + " bytes needed");
    if (n_leaves != (int)g->leaves.size() || (n_leaves && !leaves))
        return gfail(TRA_E_NULL, "expected " + std::to_string(g->leaves.size()) + " graph inputs");
    if (node == g->root && !out) return gfail(TRA_E_NULL, "the output node needs `out`");
    char *ws = (char *)workspace;
    NodeExec &e = g->ex[node];
    const GNode &nd = g->nodes[node];
    const void *in[2] = {nullptr, nullptr};
    for (size_t s = 0; s < nd.ops.size(); ++s) {
        Slot &sl = e.slot[s];
        const void *src = sl.node >= 0 ? (const void *)(ws + g->ex[sl.node].out) : leaves[sl.leaf];
        if (!src) return gfail(TRA_E_NULL, "graph input pointer is NULL");
        if (sl.repart) {
            int rc = tra_repartition(sl.bounds.data(), (int)sl.bounds.size(), sl.d_from.data(), sl.d_to.data(),
                                     sl.dtype, src, ws + sl.buf, stream);
            if (rc) return rc;
            in[s] = ws + sl.buf;
        } else {
            in[s] = src;
        }
    }
    void *scratch = e.scratch_bytes ? ws + e.scratch : nullptr;
    int rc;
    if (e.plan2) {
        rc = tra_execute(e.plan, in[0], nullptr, ws + e.lse, scratch, e.scratch_bytes, stream);
        if (rc) return rc;
        rc = tra_execute(e.plan2, in[0], ws + e.lse, ws + e.out, scratch, e.scratch_bytes, stream);
    } else {
        rc = tra_execute(e.plan, in[0], in[1], ws + e.out, scratch, e.scratch_bytes, stream);
    }
    if (rc) return rc;
    if (node == g->root) {
        std::vector<int64_t> b;
        std::vector<int32_t> dz, ones;
        for (char c : nd.out) {
            b.push_back(nd.B[(int)c]);
            dz.push_back(e.d[nd.canon.find(c)]);
            ones.push_back(1);
        }
        rc = tra_repartition(b.data(), (int)b.size(), dz.data(), ones.data(), e.out_dtype, ws + e.out, out, stream);
        if (rc) return rc;
    }
    return TRA_OK;
}

extern "C" int tra_graph_execute(tra_graph_t g, const void *const *leaves, int n_leaves, void *out, void *workspace,
                                 size_t ws_bytes, void *stream)
{
    if (!g) return gfail(TRA_E_NULL, "graph is NULL");
    for (int v = 0; v < (int)g->nodes.size(); ++v) {
        int rc = tra_graph_run_node(g, v, leaves, n_leaves, v == g->root ? out : nullptr, workspace, ws_bytes,
                                    stream);
        if (rc) return rc;
    }
    return TRA_OK;
}

extern "C" int tra_graph_destroy(tra_graph_t g)
{
    delete g;
    return TRA_OK;
}
