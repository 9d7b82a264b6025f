// choose.cpp -- partition-vector choice for an EinGraph.
//
// Page "EinDecomp：基于爱因斯坦求和与张量关系代数的自动张量并行分解算法":
//  * section 3.1: a node under d costs N*(|X sub|+|Y sub|) for its join
//    inputs plus (N/n_agg)*(n_agg-1)*|Z sub| for its aggregation (numbers
//    moved; N is the node's join-task count), and an edge costs a
//    repartition when the producer's blocking differs from what the
//    consumer needs;
//  * section 3.2: candidates must give at least P tasks and divide the
//    extents; DP[v][d_v] = Cost(v,d_v) + min over d_u of
//    (DP[u][d_u] + Repartition(d_u, d_v)), read back from the output node;
//  * section 4.3: part counts are powers of two, and the task count a
//    multiple of P.
// The repartition term is 0 when the producer's part counts on its output
// labels equal the consumer's on the matching input labels, else the size of
// the tensor.  The minimum over d_u therefore splits into "best producer
// candidate with the consumer's blocking" and "best producer candidate
// overall plus the tensor size", which keeps the DP linear in the number of
// candidates per edge while giving the same minimum and the same tie-break.
#include <algorithm>
#include <cstring>
#include <map>
#include <mutex>
#include <sstream>
#include <string>
#include <vector>

#include "graph.h"

namespace tra {

static int fail(int code, const std::string &m)
{
    set_error(m);
    return code;
}

static bool key_less(const Cand &a, int64_t ca, const Cand &b, int64_t cb)
{
    if (ca != cb) return ca < cb;
    if (a.n_tasks != b.n_tasks) return a.n_tasks < b.n_tasks;
    return a.d < b.d;
}

static int64_t einsum_cost(const std::vector<std::string> &ops, const std::string &out, const std::string &con,
                    const int64_t *B, const int32_t *D)
{
    std::string all;
    for (auto &o : ops)
        for (char c : o)
            if (all.find(c) == std::string::npos) all.push_back(c);
    int64_t n = 1, n_agg = 1;
    for (char c : all) n *= D[(int)c];
    for (char c : con) n_agg *= D[(int)c];
    auto blk = [&](const std::string &t) {
        int64_t v = 1;
        for (char c : t) v *= B[(int)c] / D[(int)c];
        return v;
    };
    int64_t in = 0;
    for (auto &o : ops) in += blk(o);
    return n * in + (n / n_agg) * (n_agg - 1) * blk(out);
}

static int64_t node_cost(const GNode &g, const Cand &c)
{
    int32_t D[128];
    for (int i = 0; i < 128; ++i) D[i] = 1;
    for (size_t i = 0; i < g.canon.size(); ++i) D[(int)g.canon[i]] = c.d[i];
    if (g.kind == "softmax") {
        // LSE over the last label, then exp(S - LSE), under the same d
        std::string hst = g.out, hs = g.out.substr(0, g.out.size() - 1), t = g.out.substr(g.out.size() - 1);
        return einsum_cost({hst}, hs, t, g.B, D) + einsum_cost({hst, hs}, hst, "", g.B, D);
    }
    return einsum_cost(g.ops, g.out, g.con, g.B, D);
}

static std::vector<std::string> split(const std::string &s, char sep)
{
    std::vector<std::string> v;
    std::string cur;
    for (char c : s) {
        if (c == sep) {
            v.push_back(cur);
            cur.clear();
        } else {
            cur.push_back(c);
        }
    }
    v.push_back(cur);
    return v;
}

int parse_graph(const char *desc, std::vector<GNode> &nodes)
{
    std::istringstream in(desc);
    std::string line;
    while (std::getline(in, line)) {
        std::istringstream ls(line);
        std::vector<std::string> f;
        std::string w;
        while (ls >> w) f.push_back(w);
        if (f.empty() || f[0][0] == '#') continue;
        if (f.size() < 5) return fail(TRA_E_GRAPH, "a node line needs 5 fields: " + line);
        GNode g;
        for (size_t o = 5; o < f.size(); ++o) {
            const std::string &kv = f[o];
            size_t eq = kv.find('=');
            if (eq == std::string::npos) return fail(TRA_E_GRAPH, "option without '=': " + kv);
            std::string k = kv.substr(0, eq), val = kv.substr(eq + 1);
            auto dt = [&](int &dst) {
                if (val == "f32") dst = D_F32;
                else if (val == "bf16") dst = D_BF16;
                else if (val == "i32") dst = D_I32;
                else return false;
                return true;
            };
            if (k == "in") {
                if (!dt(g.in_dtype)) return fail(TRA_E_GRAPH, "unknown dtype " + val);
            } else if (k == "out") {
                if (!dt(g.out_dtype)) return fail(TRA_E_GRAPH, "unknown dtype " + val);
            } else if (k == "scale") {
                g.scale = std::strtof(val.c_str(), nullptr);
            } else {
                return fail(TRA_E_GRAPH, "unknown option " + k);
            }
        }
        g.name = f[0];
        g.kind = f[1];
        g.spec = f[2];
        if (g.kind != "einsum" && g.kind != "softmax") return fail(TRA_E_GRAPH, "unknown node kind " + g.kind);
        char canon[64];
        int nl = tra_canonical_labels(g.spec.c_str(), canon, sizeof(canon));
        if (nl < 0) return nl;
        size_t arrow = g.spec.find("->");
        g.ops = split(g.spec.substr(0, arrow), ',');
        g.out = g.spec.substr(arrow + 2);
        g.canon = canon;
        g.con = g.canon.substr(g.out.size());
        if (g.kind == "softmax" && (g.ops.size() != 1 || g.ops[0] != g.out || g.out.size() < 2))
            return fail(TRA_E_GRAPH, "a softmax node is written like hst->hst");
        for (int i = 0; i < 128; ++i) g.B[i] = 0;
        for (auto &kv : split(f[3], ',')) {
            if (kv.size() < 3 || kv[1] != '=') return fail(TRA_E_GRAPH, "bad extent entry " + kv);
            long long v = std::atoll(kv.c_str() + 2);
            if (v < 1) return fail(TRA_E_GRAPH, "extent < 1 in " + kv);
            g.B[(int)kv[0]] = v;
        }
        for (char c : g.canon)
            if (!g.B[(int)c]) return fail(TRA_E_GRAPH, std::string("no extent for label '") + c + "' in " + g.name);
        g.inputs = split(f[4], ',');
        if (g.inputs.size() != g.ops.size())
            return fail(TRA_E_GRAPH, "node " + g.name + " lists " + std::to_string(g.inputs.size()) +
                                         " inputs for " + std::to_string(g.ops.size()) + " operands");
        for (size_t s = 0; s < g.inputs.size(); ++s) {
            const std::string &src = g.inputs[s];
            if (!src.empty() && src[0] == '@') {
                g.src.push_back(-1);
                continue;
            }
            int found = -1;
            for (size_t j = 0; j < nodes.size(); ++j)
                if (nodes[j].name == src) found = (int)j;
            if (found < 0) return fail(TRA_E_GRAPH, "input " + src + " of " + g.name + " is not an earlier node");
            if (nodes[found].out.size() != g.ops[s].size())
                return fail(TRA_E_GRAPH, "rank of " + src + " does not match its use in " + g.name);
            for (size_t p = 0; p < g.ops[s].size(); ++p)
                if (nodes[found].B[(int)nodes[found].out[p]] != g.B[(int)g.ops[s][p]])
                    return fail(TRA_E_GRAPH, "extents of " + src + " do not match its use in " + g.name);
            g.src.push_back(found);
        }
        nodes.push_back(g);
    }
    if (nodes.empty()) return fail(TRA_E_GRAPH, "empty graph");
    std::vector<int> uses(nodes.size(), 0);
    for (auto &g : nodes)
        for (int s : g.src)
            if (s >= 0 && ++uses[s] > 1)
                return fail(TRA_E_GRAPH, "node " + nodes[s].name + " feeds two consumers; the DP needs a tree");
    int roots = 0;
    for (size_t j = 0; j < nodes.size(); ++j) roots += uses[j] == 0;
    if (roots != 1) return fail(TRA_E_GRAPH, "the graph must have exactly one output node");
    return TRA_OK;
}

static int64_t tensor_bytes(const GNode &g, const std::string &labels, int dtype)
{
    int64_t n = dtype == D_BF16 ? 2 : 4;
    for (char l : labels) n *= g.B[(int)l];
    return n;
}

// Plan node g under candidate c.  Time model: ns = the node's own kernels'
// predicted time, plus the repartition of every graph input it needs in a
// blocking other than dense, plus, for the output node, the repartition back
// to dense.  mem = the d-dependent workspace of its step: the plans' scratch
// and the repartitioned copies of graph inputs.  False when the planner
// rejects the candidate.
static bool node_eval(const GNode &g, const Cand &c, bool is_root, int64_t &ns, int64_t &mem)
{
    std::vector<int64_t> b;
    for (char l : g.canon) b.push_back(g.B[(int)l]);
    ns = 0;
    int64_t scratch = 0;
    auto plan_ns = [&](const std::string &spec, const std::vector<int32_t> &d, const std::vector<int64_t> &bb,
                       int join, int agg, int idt, int odt, float scale) {
        tra_plan_t p = nullptr;
        if (tra_plan(spec.c_str(), bb.data(), d.data(), (int)bb.size(), join, agg, idt, odt, scale, &p)) return false;
        ns += predict_plan_ns(*p);
        scratch = std::max(scratch, (int64_t)p->info.workspace_bytes);
        tra_plan_destroy(p);
        return true;
    };
    if (g.kind == "softmax") {
        // LSE over the last label (fp32), then exp(S - LSE) in the node's out
        // dtype; as the executor runs it: one pass when the rows allow
        const std::string hst = g.out, hs = hst.substr(0, hst.size() - 1);
        tra_plan_t pl = nullptr, pn = nullptr;
        bool ok = !tra_plan((hst + "->" + hs).c_str(), b.data(), c.d.data(), (int)b.size(), TRA_JOIN_IDENT,
                            TRA_AGG_LSE, D_F32, D_F32, 1.0f, &pl) &&
                  !tra_plan((hst + "," + hs + "->" + hst).c_str(), b.data(), c.d.data(), (int)b.size(),
                            TRA_JOIN_EXP_SUB, TRA_AGG_NONE, D_F32, g.out_dtype, 1.0f, &pn);
        if (ok) {
            ns += softmax_one_pass(*pl, *pn) ? predict_softmax_one_pass_ns(*pl, *pn)
                                             : predict_plan_ns(*pl) + predict_plan_ns(*pn);
            scratch = std::max((int64_t)pl->info.workspace_bytes, (int64_t)pn->info.workspace_bytes);
        }
        tra_plan_destroy(pl);
        tra_plan_destroy(pn);
        if (!ok) return false;
    } else if (!plan_ns(g.spec, c.d, b, TRA_JOIN_MUL, TRA_AGG_SUM, g.in_dtype, g.out_dtype, g.scale)) {
        return false;
    }
    mem = scratch ? ws_round(scratch) : 0;
    auto dense = [&](const std::string &labels) {
        for (char l : labels)
            if (c.d[g.canon.find(l)] != 1) return false;
        return true;
    };
    auto elems = [&](const std::string &labels) {
        int64_t n = 1;
        for (char l : labels) n *= g.B[(int)l];
        return n;
    };
    for (size_t s = 0; s < g.src.size(); ++s)
        if (g.src[s] < 0 && !dense(g.ops[s])) {
            ns += predict_repartition_ns(elems(g.ops[s]), g.in_dtype);
            mem += ws_round(tensor_bytes(g, g.ops[s], g.in_dtype));
        }
    if (is_root && !dense(g.out)) ns += predict_repartition_ns(elems(g.out), g.out_dtype);
    return true;
}

static void make_candidates(GNode &g, int P, int model, bool is_root, int64_t mem_cap, int64_t base)
{
    const size_t L = g.canon.size();
    std::vector<std::vector<int32_t>> opts(L);
    for (size_t i = 0; i < L; ++i)
        for (int64_t k = 1; k <= g.B[(int)g.canon[i]]; k *= 2)
            if (g.B[(int)g.canon[i]] % k == 0) opts[i].push_back((int32_t)k);
    std::vector<size_t> idx(L, 0);
    while (true) {
        Cand c;
        c.d.resize(L);
        int64_t n = 1;
        for (size_t i = 0; i < L; ++i) {
            c.d[i] = opts[i][idx[i]];
            n *= c.d[i];
        }
        if (model == COST_TIME || (n >= P && n % P == 0)) {
            c.n_tasks = n;
            bool ok = true;
            if (model == COST_TIME || mem_cap > 0) {
                int64_t ns = 0;
                ok = node_eval(g, c, is_root, ns, c.mem);
                if (model == COST_TIME) c.cost = ns;
            }
            if (model != COST_TIME) c.cost = node_cost(g, c);
            if (ok && mem_cap > 0 && base + c.mem > mem_cap) ok = false;
            if (ok) g.cands.push_back(std::move(c));
        }
        size_t i = L;
        while (i > 0) {
            --i;
            if (++idx[i] < opts[i].size()) break;
            idx[i] = 0;
            if (i == 0) return;
        }
        if (L == 0) return;
    }
}

// part counts of candidate c on the labels `labels` of node g
static std::vector<int32_t> blocking(const GNode &g, const Cand &c, const std::string &labels)
{
    std::vector<int32_t> b;
    for (char l : labels) b.push_back(c.d[g.canon.find(l)]);
    return b;
}

// Memo of DP results (the EinDecomp page's closing remarks: optimise plans
// offline, load them online).  Keyed by everything the DP reads.
struct DpMemo {
    std::mutex mu;
    std::map<std::string, std::pair<std::vector<std::vector<int32_t>>, int64_t>> table;
    int64_t hits = 0, misses = 0;
};
static DpMemo &memo()
{
    static DpMemo m;
    return m;
}

static std::string dp_key(const std::vector<GNode> &nodes, int P, int model, int64_t mem_cap)
{
    std::ostringstream k;
    k << P << '|' << model << '|' << mem_cap;
    for (const GNode &g : nodes) {
        k << '\n' << g.name << ' ' << g.kind << ' ' << g.spec << ' ' << g.in_dtype << ' ' << g.out_dtype << ' '
          << g.scale;
        for (char c : g.canon) k << ' ' << c << '=' << g.B[(int)c];
        for (int s : g.src) k << ' ' << s;
    }
    return k.str();
}

int run_dp(std::vector<GNode> &nodes, int P, std::vector<std::vector<int32_t>> &d_out, int64_t &cost, int model,
           int64_t mem_cap)
{
    if (P < 1) return fail(TRA_E_GRAPH, "P must be >= 1");
    const std::string key = dp_key(nodes, P, model, mem_cap);
    {
        DpMemo &m = memo();
        std::lock_guard<std::mutex> lk(m.mu);
        auto it = m.table.find(key);
        if (it != m.table.end()) {
            m.hits++;
            d_out = it->second.first;
            cost = it->second.second;
            return TRA_OK;
        }
        m.misses++;
    }
    const int n = (int)nodes.size();
    std::vector<int> consumer(n, -1);
    for (int x = 0; x < n; ++x)
        for (int s : nodes[x].src)
            if (s >= 0) consumer[s] = x;
    // workspace live at step v whatever d is: outputs produced at or before v
    // that are read at or after v, and a softmax node's logsumexp
    std::vector<int64_t> base(n, 0);
    if (mem_cap > 0)
        for (int v = 0; v < n; ++v) {
            for (int u = 0; u <= v; ++u)
                if (u == v || consumer[u] >= v)
                    base[v] += ws_round(tensor_bytes(nodes[u], nodes[u].out, nodes[u].out_dtype));
            if (nodes[v].kind == "softmax") {
                const std::string &o = nodes[v].out;
                base[v] += ws_round(tensor_bytes(nodes[v], o.substr(0, o.size() - 1), D_F32));
            }
        }
    for (int v = 0; v < n; ++v) {
        GNode &g = nodes[v];
        make_candidates(g, P, model, consumer[v] < 0, mem_cap, base[v]);
        if (g.cands.empty())
            return fail(TRA_E_NO_CANDIDATE, mem_cap > 0 ? "no partition vector for " + g.name + " fits the memory cap"
                                                        : "no admissible partition vector for " + g.name);
    }
    for (int v = 0; v < n; ++v) {
        GNode &g = nodes[v];
        // per input slot: producer's global best and best per output blocking
        struct SlotInfo {
            int u = -1;
            int best = -1;
            std::map<std::vector<int32_t>, int> by_block;
            int64_t size = 0;
            int64_t copy_bytes = 0;
        };
        std::vector<SlotInfo> slots(g.src.size());
        for (size_t s = 0; s < g.src.size(); ++s) {
            int u = g.src[s];
            slots[s].u = u;
            if (u < 0) continue;
            GNode &pu = nodes[u];
            int64_t size = 1;
            for (char c : pu.out) size *= pu.B[(int)c];
            // the repartition term: numbers moved, or the predicted copy time
            slots[s].size = model == COST_TIME ? predict_repartition_ns(size, pu.out_dtype) : size;
            slots[s].copy_bytes = ws_round(tensor_bytes(pu, pu.out, pu.out_dtype));
            for (int i = 0; i < (int)pu.cands.size(); ++i) {
                const Cand &c = pu.cands[i];
                if (!c.feasible) continue;
                if (slots[s].best < 0 || key_less(c, c.dp, pu.cands[slots[s].best], pu.cands[slots[s].best].dp))
                    slots[s].best = i;
                auto blk = blocking(pu, c, pu.out);
                auto it = slots[s].by_block.find(blk);
                if (it == slots[s].by_block.end() ||
                    key_less(c, c.dp, pu.cands[it->second], pu.cands[it->second].dp))
                    slots[s].by_block[blk] = i;
            }
        }
        for (Cand &c : g.cands) {
            c.dp = c.cost;
            c.pick.assign(g.src.size(), -1);
            int64_t used = base[v] + c.mem;   // checked against the cap as copies are added
            for (size_t s = 0; s < g.src.size() && c.feasible; ++s) {
                if (slots[s].u < 0) continue;
                GNode &pu = nodes[slots[s].u];
                if (slots[s].best < 0) {
                    c.feasible = false;
                    break;
                }
                auto want = blocking(g, c, g.ops[s]);
                const Cand &gb = pu.cands[slots[s].best];
                const bool gb_copies = blocking(pu, gb, pu.out) != want;
                int64_t gcost = gb.dp + (gb_copies ? slots[s].size : 0);
                int pick = slots[s].best;
                int64_t pcost = gcost;
                bool copies = gb_copies;
                auto it = slots[s].by_block.find(want);
                if (it != slots[s].by_block.end()) {
                    const Cand &mb = pu.cands[it->second];
                    if (key_less(mb, mb.dp, gb, gcost) || (mem_cap > 0 && copies && used + slots[s].copy_bytes > mem_cap)) {
                        pick = it->second;
                        pcost = mb.dp;
                        copies = false;
                    }
                }
                if (copies && mem_cap > 0) {
                    if (used + slots[s].copy_bytes > mem_cap) {
                        c.feasible = false;
                        break;
                    }
                    used += slots[s].copy_bytes;
                }
                c.pick[s] = pick;
                c.dp += pcost;
            }
        }
    }
    const int root = (int)(std::find(consumer.begin(), consumer.end(), -1) - consumer.begin());
    GNode &rg = nodes[root];
    int ri = -1;
    for (int i = 0; i < (int)rg.cands.size(); ++i)
        if (rg.cands[i].feasible && (ri < 0 || key_less(rg.cands[i], rg.cands[i].dp, rg.cands[ri], rg.cands[ri].dp)))
            ri = i;
    if (ri < 0) return fail(TRA_E_NO_CANDIDATE, "no choice of partition vectors fits the memory cap");
    std::vector<int> chosen(n, -1);
    std::vector<std::pair<int, int>> stack{{root, ri}};
    while (!stack.empty()) {
        auto [v, i] = stack.back();
        stack.pop_back();
        chosen[v] = i;
        for (size_t s = 0; s < nodes[v].src.size(); ++s)
            if (nodes[v].src[s] >= 0) stack.push_back({nodes[v].src[s], nodes[v].cands[i].pick[s]});
    }
    d_out.clear();
    for (int v = 0; v < n; ++v) d_out.push_back(nodes[v].cands[chosen[v]].d);
    cost = rg.cands[ri].dp;
    DpMemo &m = memo();
    std::lock_guard<std::mutex> lk(m.mu);
    if (m.table.size() >= 256) m.table.clear();
    m.table[key] = {d_out, cost};
    return TRA_OK;
}

}  // namespace tra

using namespace tra;

extern "C" int tra_choose(const char *graph_desc, int P, int32_t *d_out, int d_cap, int64_t *cost_out)
{
    return tra_choose_ex(graph_desc, P, 0, 0, d_out, d_cap, cost_out);
}

extern "C" int tra_choose_cache_stats(int64_t *hits, int64_t *misses)
{
    DpMemo &m = memo();
    std::lock_guard<std::mutex> lk(m.mu);
    if (hits) *hits = m.hits;
    if (misses) *misses = m.misses;
    return TRA_OK;
}

extern "C" int tra_choose_cache_clear(void)
{
    DpMemo &m = memo();
    std::lock_guard<std::mutex> lk(m.mu);
    m.table.clear();
    m.hits = m.misses = 0;
    return TRA_OK;
}

extern "C" int tra_choose_ex(const char *graph_desc, int P, int flags, int64_t mem_cap_bytes, int32_t *d_out,
                             int d_cap, int64_t *cost_out)
{
    if (!graph_desc || !d_out) return fail(TRA_E_NULL, "graph_desc / d_out is NULL");
    if (flags & ~TRA_CHOOSE_TIME) return fail(TRA_E_OP, "unknown chooser flag");
    if (mem_cap_bytes < 0) return fail(TRA_E_OP, "negative memory cap");
    std::vector<GNode> nodes;
    int rc = parse_graph(graph_desc, nodes);
    if (rc) return rc;
    size_t need = 0;
    for (auto &g : nodes) need += g.canon.size();
    if ((size_t)d_cap < need) return fail(TRA_E_BUFFER, "d_out needs " + std::to_string(need) + " entries");
    std::vector<std::vector<int32_t>> ds;
    int64_t cost = 0;
    rc = run_dp(nodes, P, ds, cost, (flags & TRA_CHOOSE_TIME) ? COST_TIME : COST_PAGES, mem_cap_bytes);
    if (rc) return rc;
    size_t pos = 0;
    for (auto &dv : ds)
        for (int32_t x : dv) d_out[pos++] = x;
    if (cost_out) *cost_out = cost;
    return TRA_OK;
}
