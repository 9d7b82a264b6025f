// plan.cpp -- spec parsing, validation and the EinSum -> TRA lowering
// (page "EinDecomp：基于爱因斯坦求和与张量关系代数的自动张量并行分解算法",
// section 2.2 "from EinSum to TRA": partition the operands by d, join every
// key-matched pair of sub-tensors, aggregate by the output part of the key).
//
// On one GPU the N = prod(d) join tasks are not shipped to devices; the
// planner turns the relation layout into per-sub-dimension strides, so a
// kernel can walk any sub-tensor pair directly in HBM, and picks the kernel
// family that does the join and the aggregation of a group in registers.
#include <algorithm>
#include <initializer_list>
#include <utility>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "graph.h"
#include "plan.h"

// Matrix-core tile variants in order of preference: 4 = 256 x 256 on four
// waves with 64-deep stages and 16x16x32 products (runs of TRA_K64_RUN
// contiguous elements along each operand's staged dimension), 5 = the same
// on a 256 x 128 tile (128-wide outputs), 3 = 256 x 256 on four waves with
// 32-deep stages, 0 = 256 x 256 on eight waves, 1 = 128 x 128, 2 = 64 x 64.
#ifndef TRA_MFMA_ORDER
#define TRA_MFMA_ORDER 4, 5, 3, 0, 1, 2
#endif
// contiguous elements each operand needs along its staged dimension for the
// 64-deep tile (one 16-byte copy granule).  With runs of 64 or more every
// copy moves whole 128-byte lines; shorter runs (the attention projections
// under the pages' blockings, the four-index contraction) still measured as
// fast as or faster than the 32-deep tile.
#ifndef TRA_K64_RUN
#define TRA_K64_RUN 8
#endif

namespace tra {

static thread_local std::string g_last_error;

void set_error(const std::string &msg) { g_last_error = msg; }

static int fail(int code, const std::string &msg)
{
    set_error(msg);
    return code;
}

static bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

static int ilog2(uint64_t v)
{
    int r = 0;
    while ((1ull << r) < v) ++r;
    return r;
}

static int dtype_size(int dt) { return dt == D_BF16 ? 2 : 4; }

// Parse "ab,bc->ac" / "abc->ab".  On success fills ops / out and the
// canonical label order (output labels, then contracted by first appearance).
static int parse_spec(const char *spec, std::vector<std::string> &ops, std::string &out,
                      std::string &canon, std::string &con)
{
    if (!spec) return fail(TRA_E_NULL, "spec is NULL");
    std::string s;
    for (const char *c = spec; *c; ++c)
        if (*c != ' ') s.push_back(*c);
    size_t arrow = s.find("->");
    if (arrow == std::string::npos || s.find("->", arrow + 1) != std::string::npos)
        return fail(TRA_E_SPEC, "spec needs exactly one '->': " + s);
    std::string lhs = s.substr(0, arrow);
    out = s.substr(arrow + 2);
    ops.clear();
    size_t start = 0;
    while (true) {
        size_t comma = lhs.find(',', start);
        ops.push_back(lhs.substr(start, comma == std::string::npos ? std::string::npos : comma - start));
        if (comma == std::string::npos) break;
        start = comma + 1;
    }
    if (ops.size() < 1 || ops.size() > 2) return fail(TRA_E_SPEC, "one or two operands expected: " + s);
    auto letters = [](const std::string &t) {
        for (char c : t)
            if (!((c >= 'a' && c <= 'z') || (c >= 'A' && c <= 'Z'))) return false;
        return true;
    };
    for (auto &o : ops) {
        if (o.empty()) return fail(TRA_E_SPEC, "an operand has no labels: " + s);
        if (!letters(o)) return fail(TRA_E_SPEC, "labels must be letters: " + s);
    }
    if (!letters(out)) return fail(TRA_E_SPEC, "labels must be letters: " + s);
    auto repeated = [](const std::string &t) {
        for (size_t i = 0; i < t.size(); ++i)
            if (t.find(t[i], i + 1) != std::string::npos) return true;
        return false;
    };
    for (auto &o : ops)
        if (repeated(o)) return fail(TRA_E_LABELS, "label repeated within an operand: " + s);
    if (repeated(out)) return fail(TRA_E_LABELS, "label repeated in the output: " + s);
    for (auto &o : ops)
        if ((int)o.size() > kMaxRank) return fail(TRA_E_LABELS, "rank above 12: " + s);
    if ((int)out.size() > kMaxRank) return fail(TRA_E_LABELS, "rank above 12: " + s);
    std::string all = ops[0] + (ops.size() > 1 ? ops[1] : "");
    for (char c : out)
        if (all.find(c) == std::string::npos)
            return fail(TRA_E_LABELS, std::string("output label '") + c + "' is in no operand");
    con.clear();
    for (char c : all)
        if (out.find(c) == std::string::npos && con.find(c) == std::string::npos) con.push_back(c);
    canon = out + con;
    if ((int)canon.size() > kMaxLabels) return fail(TRA_E_LABELS, "more than 24 labels");
    return TRA_OK;
}

// Relation-layout strides of a tensor with labels `t`: in-block stride of
// each label (row-major over block extents) and key stride (row-major over
// part counts, times the block volume).
void relation_strides(const std::string &t, const int64_t *B, const int32_t *d, int64_t *bs, int64_t *ks)
{
    int64_t vol = 1;
    for (char c : t) vol *= B[(int)c] / d[(int)c];
    int64_t sb = 1, sk = vol;
    for (int p = (int)t.size() - 1; p >= 0; --p) {
        int c = t[p];
        bs[p] = sb;
        ks[p] = sk;
        sb *= B[c] / d[c];
        sk *= d[c];
    }
}

// Sub-dimensions of a label group: keys first (in group order), then the
// in-block indices; `tens` are up to three tensors whose strides are recorded.
static std::vector<SubDim> group_subdims(const std::string &group, const int64_t *B, const int32_t *d,
                                         const std::string *tens[3])
{
    std::vector<SubDim> v;
    for (int pass = 0; pass < 2; ++pass) {
        for (char c : group) {
            int64_t ext = pass == 0 ? d[(int)c] : B[(int)c] / d[(int)c];
            if (ext == 1) continue;
            SubDim s{(uint32_t)ext, {0, 0, 0}};
            for (int t = 0; t < 3; ++t) {
                if (!tens[t]) continue;
                size_t p = tens[t]->find(c);
                if (p == std::string::npos) continue;
                int64_t bs[kMaxRank], ks[kMaxRank];
                relation_strides(*tens[t], B, d, bs, ks);
                s.st[t] = pass == 0 ? ks[p] : bs[p];
            }
            v.push_back(s);
        }
    }
    return v;
}

static Radix to_radix(const std::vector<SubDim> &v)
{
    Radix r{};
    r.n = (int32_t)v.size();
    for (size_t i = 0; i < v.size(); ++i) {
        r.ext[i] = v[i].ext;
        for (int t = 0; t < 3; ++t) r.st[t][i] = v[i].st[t];
    }
    return r;
}

bool to_pow2(const std::vector<SubDim> &v, Pow2Group &g)
{
    g = Pow2Group{};
    if ((int)v.size() > kP2Max) return false;
    g.n = (int32_t)v.size();
    int sh = 0;
    uint64_t total = 1;
    for (int i = (int)v.size() - 1; i >= 0; --i) {
        if (!is_pow2(v[i].ext)) return false;
        g.sh[i] = (uint32_t)sh;
        g.mask[i] = v[i].ext - 1;
        for (int t = 0; t < 3; ++t) g.st[t][i] = (int32_t)v[i].st[t];
        sh += ilog2(v[i].ext);
        total *= v[i].ext;
    }
    if (total > 0x7fffffffull) return false;
    g.total = (uint32_t)total;
    return true;
}

static int64_t elems_of(const std::string &t, const int64_t *B)
{
    int64_t n = 1;
    for (char c : t) n *= B[(int)c];
    return n;
}

// Last sub-dimension of a group has stride 1 in tensor t and a multiple of vec elements.
static bool contiguous_last(const std::vector<SubDim> &v, int t, int vec)
{
    return !v.empty() && v.back().st[t] == 1 && v.back().ext % vec == 0;
}

// Largest offset a list of sub-dimension groups can reach in tensor slot t of
// each group (the kernels never index beyond it).  Checked against the
// tensor's element count before any launch.
static int64_t max_offset(std::initializer_list<std::pair<const std::vector<SubDim> *, int>> groups)
{
    int64_t m = 0;
    for (auto &g : groups)
        for (const SubDim &s : *g.first) m += (int64_t)(s.ext - 1) * s.st[g.second];
    return m;
}

static void choose_split(tra_plan_s &p, int64_t tiles, int64_t k_steps, int bk)
{
    int split = 1;
    if (tiles < 128) {
        while (split * 2 <= k_steps && tiles * split < 256 && k_steps % (split * 2) == 0) split *= 2;
    }
    p.gv.split = split;
    p.gv.k_per_split = (int32_t)(k_steps / split * bk);
    p.info.agg_split = split;
    p.info.workspace_bytes = split > 1 ? (size_t)split * (size_t)p.info.z_elems * 4 : 0;
}

// Try the tile kernels (GEMM view).  Returns true and fills p when eligible.
// Output labels of a two-operand product split into its batch (in both
// operands), row (X only) and column (Y only) groups, in output order.
static void tile_groups(const tra_plan_s &p, std::string &M, std::string &N, std::string &Bt)
{
    for (char c : p.zl) {
        bool inx = p.xl.find(c) != std::string::npos, iny = p.yl.find(c) != std::string::npos;
        if (inx && iny) Bt.push_back(c);
        else if (inx) M.push_back(c);
        else N.push_back(c);
    }
}

// Z's four consecutive output columns, from a multiple of 4, are one aligned
// vector: the column group's lowest digit has Z stride 1 and covers at least
// two bits, and every other Z stride (rows, the other column digits, the
// batch) is a multiple of 4 elements.
static bool z_vec4(const GemmView &gv)
{
    bool low = false;
    for (int i = 0; i < kP2Max; ++i) {
        if (!gv.gn.mask[i]) continue;
        if (gv.gn.sh[i] == 0) {
            if (gv.gn.st[1][i] != 1 || gv.gn.mask[i] < 3) return false;
            low = true;
        } else if (gv.gn.st[1][i] % 4) {
            return false;
        }
    }
    for (int i = 0; i < kP2Max; ++i) {
        if (gv.gm.mask[i] && gv.gm.st[1][i] % 4) return false;
        if (gv.gb.mask[i] && gv.gb.st[2][i] % 4) return false;
    }
    return low;
}

// k-tile depth of the vector-ALU tile kernel (masked edge tiles need whole k-tiles)
constexpr int64_t VT_BK_RAGGED = 32;

static bool lower_tile(tra_plan_s &p)
{
    if (p.n_ops != 2) return false;
    const std::string &X = p.xl, &Y = p.yl, &Z = p.zl;
    std::string M, N, Bt, K;
    tile_groups(p, M, N, Bt);
    for (char c : p.con) {
        bool inx = X.find(c) != std::string::npos, iny = Y.find(c) != std::string::npos;
        if (!(inx && iny)) return false;  // contracted label in one operand only
        K.push_back(c);
    }
    if (M.empty() || N.empty() || K.empty()) return false;
    const std::string *tm[3] = {&X, &Z, nullptr}, *tn[3] = {&Y, &Z, nullptr};
    const std::string *tk[3] = {&X, &Y, nullptr}, *tb[3] = {&X, &Y, &Z};
    auto sm = group_subdims(M, p.B, p.d, tm), sn = group_subdims(N, p.B, p.d, tn);
    auto sk = group_subdims(K, p.B, p.d, tk), sb = group_subdims(Bt, p.B, p.d, tb);
    GemmView gv{};
    const bool pm = to_pow2(sm, gv.gm), pn = to_pow2(sn, gv.gn);
    if (!to_pow2(sk, gv.gk) || !to_pow2(sb, gv.gb)) return false;
    gv.post_scale = p.post_scale;
    gv.z_elems = p.info.z_elems;
    const bool mfma = p.join == J_MUL && p.agg == A_SUM && p.in_dtype == D_BF16;
    // join / aggregate pairs the vector-ALU tile kernel is built for
    const bool valu_op = (p.join == J_MUL && p.agg == A_SUM) || (p.join == J_SQDIFF && p.agg == A_SUM) ||
                         (p.join == J_ADD && (p.agg == A_MAX || p.agg == A_MIN));
    const bool valu = valu_op && (p.in_dtype == D_F32 || p.in_dtype == D_I32);
    if (!mfma && !valu) return false;
    if (max_offset({{&sm, 0}, {&sk, 0}, {&sb, 0}}) >= p.info.x_elems ||
        max_offset({{&sn, 0}, {&sk, 1}, {&sb, 1}}) >= p.info.y_elems ||
        max_offset({{&sm, 1}, {&sn, 1}, {&sb, 2}}) >= p.info.z_elems)
        return false;  // never true for a valid relation layout
    const int vec = mfma ? 8 : 4;
    bool ak, bk;
    if (contiguous_last(sk, 0, vec)) ak = true;
    else if (contiguous_last(sm, 0, vec)) ak = false;
    else return false;
    if (contiguous_last(sk, 1, vec)) bk = true;
    else if (contiguous_last(sn, 0, vec)) bk = false;
    else return false;
    // pick the first tile variant, in order of preference, that divides the problem
    static const int kMfmaOrder[] = {TRA_MFMA_ORDER};
    constexpr int kMfmaVariants = sizeof(kMfmaOrder) / sizeof(kMfmaOrder[0]);
    // the 64-deep tile: each operand K-major or MN-major with TRA_K64_RUN
    // contiguous elements along its staged dimension
    const bool k64 = ((ak && contiguous_last(sk, 0, TRA_K64_RUN)) || (!ak && contiguous_last(sm, 0, TRA_K64_RUN))) &&
                     ((bk && contiguous_last(sk, 1, TRA_K64_RUN)) || (!bk && contiguous_last(sn, 0, TRA_K64_RUN)));
    for (int n = 0; n < (mfma ? kMfmaVariants : 4) && pm && pn; ++n) {
        const int variant = mfma ? kMfmaOrder[n] : n;
        if (mfma && (variant == 4 || variant == 5) && !k64) continue;
        TileShape ts = mfma ? mfma_tile_shape(variant) : valu_tile_shape(variant);
        if (ts.bm == 0) break;
        if (gv.gm.total % ts.bm || gv.gn.total % ts.bn || gv.gk.total % ts.bk) continue;
        p.gv = gv;
        p.gv.z_vec4 = z_vec4(gv) ? 1 : 0;
        p.tile = variant;
        p.a_kmajor = ak;
        p.b_kmajor = bk;
        p.kernel = mfma ? TRA_KERNEL_MFMA_BF16 : TRA_KERNEL_VALU_TILE;
        int64_t tiles = (int64_t)(gv.gm.total / ts.bm) * (gv.gn.total / ts.bn) * gv.gb.total;
        choose_split(p, tiles, gv.gk.total / ts.bk, ts.bk);
        if (!mfma && p.in_dtype == D_I32 && p.join == J_ADD && (p.agg == A_MAX || p.agg == A_MIN)) {
            // int32 max-plus / min-plus: the packed 16-bit kernel behind a
            // range check whose flags live in the workspace
            p.tile = 1;
            p.info.workspace_bytes = small_int_flags_offset(p.gv.split, p.info.z_elems) + SMALL_INT_FLAG_BYTES;
        }
        return true;
    }
    // Masked edge tiles (vector-ALU joins): output rows and columns of any
    // extent and digit structure, addressed by mixed radix, the last tile row
    // and column partly out of range; the contracted range keeps whole
    // power-of-two k-tiles, so every term of every output is a real one.
    if (!mfma && gv.gk.total % VT_BK_RAGGED == 0) {
        int64_t M = 1, N = 1;
        for (auto &d : sm) M *= d.ext;
        for (auto &d : sn) N *= d.ext;
        if (M < 4 || N < 4 || M >= ((int64_t)1 << 31) || N >= ((int64_t)1 << 31)) return false;
        TileShape ts = valu_tile_shape(0);
        gv.gm = Pow2Group{};
        gv.gn = Pow2Group{};
        gv.gm.total = (uint32_t)((M + ts.bm - 1) / ts.bm * ts.bm);
        gv.gn.total = (uint32_t)((N + ts.bn - 1) / ts.bn * ts.bn);
        p.gv = gv;
        p.tile = 0;
        p.a_kmajor = ak;
        p.b_kmajor = bk;
        p.ragged = true;
        p.rag.m = to_radix(sm);
        p.rag.n = to_radix(sn);
        p.rag.M = (uint32_t)M;
        p.rag.N = (uint32_t)N;
        p.kernel = TRA_KERNEL_VALU_TILE;
        int64_t tiles = (int64_t)(gv.gm.total / ts.bm) * (gv.gn.total / ts.bn) * gv.gb.total;
        choose_split(p, tiles, gv.gk.total / ts.bk, ts.bk);
        return true;
    }
    return false;
}

// The output of a join over an empty contracted range (an operand with no
// elements): the generic kernel with no contracted digits reads nothing and
// writes post_scale times the aggregate's identity to every output element.
static bool lower_identity(tra_plan_s &p)
{
    const std::string *tz[3] = {nullptr, nullptr, nullptr};
    auto so = group_subdims(p.zl, p.B, p.d, tz);
    p.gen = GenericDesc{};
    p.gen.out = to_radix(so);
    p.gen.n_out = p.info.z_elems;
    p.gen.n_con = 0;
    p.gen.post_scale = p.post_scale;
    p.kernel = TRA_KERNEL_GENERIC;
    return true;
}

// Plans with at most this many outputs and at least this many contracted
// terms per output take the split reduction (see lower_generic).
constexpr int64_t kSplitReduceMaxOut = 4096;
constexpr int64_t kSplitReduceMinTerms = 4096;

static bool lower_generic(tra_plan_s &p)
{
    const std::string *tz[3] = {&p.xl, p.n_ops == 2 ? &p.yl : nullptr, nullptr};
    auto so = group_subdims(p.zl, p.B, p.d, tz);
    auto sc = group_subdims(p.con, p.B, p.d, tz);
    if (max_offset({{&so, 0}, {&sc, 0}}) >= p.info.x_elems ||
        (p.n_ops == 2 && max_offset({{&so, 1}, {&sc, 1}}) >= p.info.y_elems))
        return false;
    p.gen.out = to_radix(so);
    p.gen.con = to_radix(sc);
    p.gen.n_out = p.info.z_elems;
    int64_t nc = 1;
    for (auto &s : sc) nc *= s.ext;
    p.gen.n_con = nc;
    p.gen.post_scale = p.post_scale;
    p.kernel = TRA_KERNEL_GENERIC;

    if (p.agg == A_NONE) {
        p.el.out = p.gen.out;
        p.el.n_out = p.gen.n_out;
        p.el.post_scale = p.post_scale;
        // vectorise along the fastest output sub-dimension when it is
        // contiguous (stride 1) or broadcast (stride 0) in both operands
        int vec = 1;
        if (!so.empty()) {
            const SubDim &f = so.back();
            bool okx = f.st[0] == 1 || f.st[0] == 0;
            bool oky = p.n_ops == 1 || f.st[1] == 1 || f.st[1] == 0;
            if (okx && oky && f.ext % 4 == 0) vec = 4;
        }
        p.el.vec = vec;
        p.el.p2 = 0;
        if (vec == 4 && so.back().st[0] == 1 && p.info.z_elems < (int64_t)1 << 31 && to_pow2(so, p.el.out_p2)) {
            p.el.p2 = 1;
            p.el.y_step = p.n_ops == 2 ? (int32_t)so.back().st[1] : 0;
        }
        p.kernel = TRA_KERNEL_ELEMWISE;
        return true;
    }
    // Few outputs and a long contracted range: one thread (or one wavefront)
    // per output would leave the chip idle.  Cut each output's range into
    // chunks folded by whole workgroups (four waves, combined in order), and
    // fold the chunks' partials in order in a second pass: enough chunks for
    // ~2048 workgroups, each chunk at least 4096 terms.
    if (p.gen.n_out <= kSplitReduceMaxOut && p.gen.n_con >= kSplitReduceMinTerms && !sc.empty()) {
        int64_t split = 1;
        while (split < 1024 && split * 2 * p.gen.n_out <= 2048 && p.gen.n_con / (split * 2) >= kSplitReduceMinTerms)
            split *= 2;
        p.gen.split = (int32_t)split;
        p.gen.chunk = (p.gen.n_con + split - 1) / split;
        p.info.agg_split = split;
        p.info.workspace_bytes = split > 1 ? (size_t)split * (size_t)p.gen.n_out * 4 : 0;
    }
    // one wavefront per output row when the last contracted run is contiguous in
    // X and contiguous or broadcast in Y (a Y strided along the run makes every
    // wavefront touch one cache line per lane; one thread per output element
    // then reads Y coalesced across the wavefront and is measured 5x faster)
    if (!sc.empty() && sc.back().st[0] == 1 && sc.back().ext >= 64 &&
        (p.n_ops == 1 || sc.back().st[1] == 0 || sc.back().st[1] == 1)) {
        std::vector<SubDim> outer(sc.begin(), sc.end() - 1);
        p.row.out = p.gen.out;
        p.row.outer = to_radix(outer);
        p.row.n_out = p.gen.n_out;
        int64_t no = 1;
        for (auto &s : outer) no *= s.ext;
        p.row.n_outer = no;
        p.row.inner = sc.back().ext;
        p.row.inner_sy = sc.back().st[1];
        p.row.post_scale = p.post_scale;
        p.row.p2 = 0;
        const int64_t sy = sc.back().st[1];
        if (p.row.inner % 256 == 0 && (p.n_ops == 1 || sy == 0 || sy == 1) && to_pow2(so, p.row.out_p2) &&
            to_pow2(outer, p.row.outer_p2))
            p.row.p2 = 1;
        p.kernel = TRA_KERNEL_ROWREDUCE;
    }
    return true;
}

}  // namespace tra

using namespace tra;

extern "C" {

const char *tra_last_error(void) { return g_last_error.c_str(); }

const char *tra_status_string(int s)
{
    switch (s) {
    case TRA_OK: return "ok";
    case TRA_E_NULL: return "null pointer argument";
    case TRA_E_SPEC: return "spec does not parse";
    case TRA_E_LABELS: return "invalid labels";
    case TRA_E_INDIVISIBLE: return "part count does not divide the extent";
    case TRA_E_DLEN: return "wrong partition vector / label count";
    case TRA_E_DTYPE: return "unsupported dtype";
    case TRA_E_OP: return "invalid join / aggregate";
    case TRA_E_WORKSPACE: return "workspace too small";
    case TRA_E_ALIGN: return "device pointer not 16-byte aligned";
    case TRA_E_HIP: return "HIP runtime error";
    case TRA_E_NO_CANDIDATE: return "no admissible partition vector";
    case TRA_E_RANGE: return "tensor too large";
    case TRA_E_GRAPH: return "malformed graph description";
    case TRA_E_BUFFER: return "output buffer too small";
    }
    return "unknown status";
}

int tra_canonical_labels(const char *spec, char *out, int out_cap)
{
    if (!out) return fail(TRA_E_NULL, "out is NULL");
    std::vector<std::string> ops;
    std::string zl, canon, con;
    int rc = parse_spec(spec, ops, zl, canon, con);
    if (rc) return rc;
    if ((int)canon.size() + 1 > out_cap) return fail(TRA_E_BUFFER, "label buffer too small");
    std::memcpy(out, canon.c_str(), canon.size() + 1);
    return (int)canon.size();
}

int tra_d_from_operand_form(const char *spec, const int32_t *d_ops, int n_ops, int32_t *d_out, int d_out_cap)
{
    if (!d_ops || !d_out) return fail(TRA_E_NULL, "NULL vector");
    std::vector<std::string> ops;
    std::string zl, canon, con;
    int rc = parse_spec(spec, ops, zl, canon, con);
    if (rc) return rc;
    int occ = 0;
    for (auto &o : ops) occ += (int)o.size();
    if (n_ops != occ) return fail(TRA_E_DLEN, "per-operand vector needs one entry per label occurrence");
    if (d_out_cap < (int)canon.size()) return fail(TRA_E_BUFFER, "d_out too small");
    int32_t seen[128];
    for (int i = 0; i < 128; ++i) seen[i] = 0;
    int pos = 0;
    for (auto &o : ops)
        for (char c : o) {
            int32_t v = d_ops[pos++];
            if (seen[(int)c] && seen[(int)c] != v)
                return fail(TRA_E_DLEN, std::string("occurrences of label '") + c + "' are split differently");
            seen[(int)c] = v;
        }
    for (size_t i = 0; i < canon.size(); ++i) d_out[i] = seen[(int)canon[i]];
    return TRA_OK;
}

static int validate_bounds(const std::string &canon, const int64_t *bounds, const int32_t *d, int n_labels,
                           int64_t *B, int32_t *D)
{
    if (!bounds || !d) return fail(TRA_E_NULL, "bounds / d is NULL");
    if (n_labels != (int)canon.size())
        return fail(TRA_E_DLEN, "expected " + std::to_string(canon.size()) + " labels (" + canon + "), got " +
                                    std::to_string(n_labels));
    for (int i = 0; i < n_labels; ++i) {
        int c = canon[i];
        if (bounds[i] < 0) return fail(TRA_E_INDIVISIBLE, std::string("extent of '") + (char)c + "' < 0");
        if (bounds[i] == 0 && d[i] != 1)
            return fail(TRA_E_INDIVISIBLE, std::string("a zero extent ('") + (char)c + "') takes d = 1");
        if (d[i] < 1 || (bounds[i] > 0 && bounds[i] % d[i]))
            return fail(TRA_E_INDIVISIBLE, std::string("d of '") + (char)c + "' = " + std::to_string(d[i]) +
                                               " does not divide " + std::to_string(bounds[i]));
        B[c] = bounds[i];
        D[c] = d[i];
    }
    return TRA_OK;
}

int tra_cost(const char *spec, const int64_t *bounds, const int32_t *d, int n_labels, int64_t *cost_out)
{
    if (!cost_out) return fail(TRA_E_NULL, "cost_out is NULL");
    std::vector<std::string> ops;
    std::string zl, canon, con;
    int rc = parse_spec(spec, ops, zl, canon, con);
    if (rc) return rc;
    int64_t B[128] = {0};
    int32_t D[128] = {0};
    rc = validate_bounds(canon, bounds, d, n_labels, B, D);
    if (rc) return rc;
    int64_t n = 1, n_agg = 1;
    for (char c : canon) n *= D[(int)c];
    for (char c : con) n_agg *= D[(int)c];
    auto blk = [&](const std::string &t) {
        int64_t v = 1;
        for (char c : t) v *= B[(int)c] / D[(int)c];
        return v;
    };
    int64_t in = 0;
    for (auto &o : ops) in += blk(o);
    *cost_out = n * in + (n / n_agg) * (n_agg - 1) * blk(zl);
    return TRA_OK;
}

int tra_plan(const char *spec, const int64_t *bounds, const int32_t *d, int n_labels, int join_op, int agg_op,
             int in_dtype, int out_dtype, float post_scale, tra_plan_t *out_plan)
{
    if (!out_plan) return fail(TRA_E_NULL, "out_plan is NULL");
    *out_plan = nullptr;
    std::vector<std::string> ops;
    std::string zl, canon, con;
    int rc = parse_spec(spec, ops, zl, canon, con);
    if (rc) return rc;
    tra_plan_s *p = new (std::nothrow) tra_plan_s();
    if (!p) return fail(TRA_E_RANGE, "out of host memory");
    rc = validate_bounds(canon, bounds, d, n_labels, p->B, p->d);
    if (rc) {
        delete p;
        return rc;
    }
    auto bad = [&](int code, const std::string &m) {
        delete p;
        return fail(code, m);
    };
    if (in_dtype < D_F32 || in_dtype > D_I32 || out_dtype < D_F32 || out_dtype > D_I32)
        return bad(TRA_E_DTYPE, "unknown dtype");
    if (join_op < J_MUL || join_op > J_SUB) return bad(TRA_E_OP, "unknown join");
    if (agg_op < A_NONE || agg_op > A_LSE) return bad(TRA_E_OP, "unknown aggregate");
    if (agg_op == A_NONE && !con.empty()) return bad(TRA_E_OP, "aggregate NONE with contracted labels " + con);
    if (ops.size() == 1 && join_op != J_IDENT) return bad(TRA_E_OP, "a one-operand spec takes the ident join");
    if (ops.size() == 2 && join_op == J_IDENT) return bad(TRA_E_OP, "ident takes one operand");
    const bool is_int = in_dtype == D_I32;
    if (is_int && (join_op == J_EXP_SUB || agg_op == A_LSE)) return bad(TRA_E_DTYPE, "exp / lse on integers");
    if (is_int != (out_dtype == D_I32)) return bad(TRA_E_DTYPE, "integer inputs give integer outputs only");
    if (is_int && post_scale != 1.0f) return bad(TRA_E_OP, "post_scale applies to floats only");

    p->spec = spec;
    p->n_ops = (int)ops.size();
    p->xl = ops[0];
    p->yl = ops.size() > 1 ? ops[1] : "";
    p->zl = zl;
    p->canon = canon;
    p->con = con;
    p->join = join_op;
    p->agg = agg_op;
    p->in_dtype = in_dtype;
    p->out_dtype = out_dtype;
    p->post_scale = post_scale;

    tra_plan_info_t &in = p->info;
    in.n_tasks = 1;
    in.n_agg = 1;
    for (char c : canon) in.n_tasks *= p->d[(int)c];
    for (char c : con) in.n_agg *= p->d[(int)c];
    in.n_groups = in.n_tasks / in.n_agg;
    in.agg_split = 1;
    in.x_elems = elems_of(p->xl, p->B);
    in.y_elems = p->n_ops == 2 ? elems_of(p->yl, p->B) : 0;
    in.z_elems = elems_of(zl, p->B);
    for (int64_t e : {in.x_elems, in.y_elems, in.z_elems})
        if (e >= (int64_t)1 << 31) return bad(TRA_E_RANGE, "a tensor has 2^31 or more elements");
    in.x_bytes = (size_t)in.x_elems * dtype_size(in_dtype);
    in.y_bytes = (size_t)in.y_elems * dtype_size(in_dtype);
    in.z_bytes = (size_t)in.z_elems * dtype_size(out_dtype);
    in.workspace_bytes = 0;
    in.n_labels = (int32_t)canon.size();
    std::memset(in.labels, 0, sizeof(in.labels));
    std::memcpy(in.labels, canon.c_str(), canon.size());

    if (in.z_elems == 0) {
        p->kernel = TRA_KERNEL_EMPTY;   // nothing to compute
    } else if (in.x_elems == 0 || (p->n_ops == 2 && in.y_elems == 0)) {
        // an empty contracted range: every output element is the aggregate's identity
        if (!lower_identity(*p)) return bad(TRA_E_RANGE, "internal: descriptor exceeds a tensor");
    } else if (!lower_tile(*p) && !lower_generic(*p)) {
        return bad(TRA_E_RANGE, "internal: descriptor exceeds a tensor");
    }
    in.kernel = p->kernel;
    in.tile = p->kernel == TRA_KERNEL_MFMA_BF16 || p->kernel == TRA_KERNEL_VALU_TILE ? p->tile : -1;
    *out_plan = p;
    return TRA_OK;
}

int tra_plan_info(tra_plan_t plan, tra_plan_info_t *info)
{
    if (!plan || !info) return fail(TRA_E_NULL, "plan / info is NULL");
    *info = plan->info;
    return TRA_OK;
}

int tra_plan_destroy(tra_plan_t plan)
{
    delete plan;
    return TRA_OK;
}

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int tra_execute(tra_plan_t p, const void *x, const void *y, void *z, void *ws, size_t ws_bytes, void *stream)
{
    if (!p) return fail(TRA_E_NULL, "plan is NULL");
    // pointers of tensors with no elements may be NULL
    if ((!x && p->info.x_elems) || (!z && p->info.z_elems) || (p->n_ops == 2 && !y && p->info.y_elems))
        return fail(TRA_E_NULL, "operand / output pointer is NULL");
    if (!aligned16(x) || !aligned16(z) || (y && !aligned16(y)) || (ws && !aligned16(ws)))
        return fail(TRA_E_ALIGN, "device pointers must be 16-byte aligned");
    if (p->info.workspace_bytes > 0 && (!ws || ws_bytes < p->info.workspace_bytes))
        return fail(TRA_E_WORKSPACE, "workspace of " + std::to_string(p->info.workspace_bytes) + " bytes needed");
    if (p->kernel == TRA_KERNEL_EMPTY) return TRA_OK;
    int err = 0;
    switch (p->kernel) {
    case TRA_KERNEL_MFMA_BF16: err = launch_mfma_bf16(*p, x, y, z, ws, stream); break;
    case TRA_KERNEL_VALU_TILE: err = launch_valu_tile(*p, x, y, z, ws, stream); break;
    case TRA_KERNEL_ROWREDUCE: err = launch_rowreduce(*p, x, y, z, ws, stream); break;
    case TRA_KERNEL_ELEMWISE: err = launch_elemwise(*p, x, y, z, stream); break;
    default: err = launch_generic(*p, x, y, z, ws, stream); break;
    }
    if (err) return fail(TRA_E_HIP, std::string("kernel launch failed: ") + hip_error_text(err));
    return TRA_OK;
}

int tra_execute_chain(tra_plan_t a, tra_plan_t b, const void *xa, const void *ya, const void *xb, void *z,
                      void *stream)
{
    if (!a || !b) return fail(TRA_E_NULL, "plan is NULL");
    if (!elemwise_chainable(*a, *b))
        return fail(TRA_E_OP, "the plans do not chain: both must be elementwise (aggregate none) over the same "
                              "output relation, the second plan's second operand laid out as its output, "
                              "float dtypes with the second plan's input dtype the first plan's output dtype");
    if (a->info.z_elems && (!xa || !xb || !z || (a->n_ops == 2 && !ya && a->info.y_elems)))
        return fail(TRA_E_NULL, "operand / output pointer is NULL");
    if (!aligned16(xa) || !aligned16(xb) || !aligned16(z) || (ya && !aligned16(ya)))
        return fail(TRA_E_ALIGN, "device pointers must be 16-byte aligned");
    int err = launch_elemwise_chain(*a, *b, xa, ya, xb, z, stream);
    if (err) return fail(TRA_E_HIP, std::string("kernel launch failed: ") + hip_error_text(err));
    return TRA_OK;
}

int tra_execute_contract_chain(tra_plan_t c, tra_plan_t a, tra_plan_t b, const void *xc, const void *yc,
                               const void *ya, const void *xb, void *z, void *stream)
{
    if (!c || !a || !b) return fail(TRA_E_NULL, "plan is NULL");
    if (c->kernel != TRA_KERNEL_MFMA_BF16 || c->gv.split != 1 || c->out_dtype != D_F32)
        return fail(TRA_E_OP, "the product must run on the matrix-core kernel with no split of its contracted "
                              "range and an fp32 output");
    if (a->kernel != TRA_KERNEL_ELEMWISE || b->kernel != TRA_KERNEL_ELEMWISE || a->n_ops != 2 || b->n_ops != 2)
        return fail(TRA_E_OP, "both steps must be two-operand elementwise plans (aggregate none)");
    if (a->in_dtype != D_F32 || (a->out_dtype != D_F32 && a->out_dtype != D_BF16) || b->in_dtype != a->out_dtype ||
        b->out_dtype != a->out_dtype)
        return fail(TRA_E_OP, "dtypes: the first step reads fp32, and its output, the second step's input and "
                              "the result share one dtype, bf16 or fp32");
    const std::string &Z = c->zl;
    if (a->xl != Z || a->zl != Z || b->xl != Z || b->yl != Z || b->zl != Z)
        return fail(TRA_E_OP, "the product's output, the first step's first operand and output, and both "
                              "operands and the output of the second step must be one relation (same labels "
                              "in the same order)");
    for (char ch : Z)
        if (a->B[(int)ch] != c->B[(int)ch] || b->B[(int)ch] != c->B[(int)ch] || a->d[(int)ch] != c->d[(int)ch] ||
            b->d[(int)ch] != c->d[(int)ch])
            return fail(TRA_E_OP, "the three plans must agree on the output's extents and d");
    for (char ch : a->yl)
        if (Z.find(ch) == std::string::npos)
            return fail(TRA_E_OP, "the first step's second operand may only carry output labels");
    if (c->info.z_elems && (!xc || !yc || !ya || !xb || !z)) return fail(TRA_E_NULL, "operand / output pointer is NULL");
    if (!aligned16(xc) || !aligned16(yc) || !aligned16(ya) || !aligned16(xb) || !aligned16(z))
        return fail(TRA_E_ALIGN, "device pointers must be 16-byte aligned");
    if (c->info.z_elems == 0) return TRA_OK;
    std::string M, N, Bt;
    tile_groups(*c, M, N, Bt);
    const std::string *tr[3] = {&a->yl, nullptr, nullptr};
    ChainEpi ce{};
    if (!to_pow2(group_subdims(Bt, c->B, c->d, tr), ce.rb) || !to_pow2(group_subdims(M, c->B, c->d, tr), ce.rm) ||
        !to_pow2(group_subdims(N, c->B, c->d, tr), ce.rn))
        return fail(TRA_E_OP, "the first step's second operand has no power-of-two digit layout");
    ce.ya = ya;
    ce.xb = xb;
    ce.join_a = a->join;
    ce.join_b = b->join;
    ce.scale_a = a->el.post_scale;
    ce.scale_b = b->el.post_scale;
    int err = launch_mfma_chain(*c, ce, a->out_dtype == D_F32, xc, yc, z, stream);
    if (err) return fail(TRA_E_HIP, std::string("kernel launch failed: ") + hip_error_text(err));
    return TRA_OK;
}

// Digits of a re-blocking: the layout with part counts `de` is enumerated
// (key digits of every label, then in-block digits) and each digit carries its
// stride in the layout with part counts `ds`.  For each label the enumerated
// digits are refined so that every refined digit maps to the other layout
// affinely:
//  * b_s % b_e == 0 (enumerated block inside the other's block, per = b_s/b_e):
//      k_e = q*per + p  ->  k_s = q, r_s = p*b_e + r_e
//  * b_e % b_s == 0 (the other's block inside the enumerated block, per = b_e/b_s):
//      r_e = p*b_s + s  ->  k_s = k_e*per + p, r_s = s
// The refined digits sit where the original digit sat, so the enumeration
// order is unchanged.  Neighbours that are one affine run in the other layout
// are merged.  False when, for some label, neither block extent divides the
// other.
static bool rep_subdims(const std::string &t, const int64_t *B, const int32_t *ds, const int32_t *de,
                        std::vector<SubDim> &merged)
{
    int64_t bss[kMaxRank], kss[kMaxRank];
    relation_strides(t, B, ds, bss, kss);
    std::vector<SubDim> keys, inner;
    for (size_t i = 0; i < t.size(); ++i) {
        int c = t[i];
        int64_t bs = B[c] / ds[c], be = B[c] / de[c];
        if (bs % be == 0) {
            int64_t per = bs / be;
            if (ds[c] > 1) keys.push_back({(uint32_t)ds[c], {kss[i], 0, 0}});
            if (per > 1) keys.push_back({(uint32_t)per, {be * bss[i], 0, 0}});
            if (be > 1) inner.push_back({(uint32_t)be, {bss[i], 0, 0}});
        } else if (be % bs == 0) {
            int64_t per = be / bs;
            if (de[c] > 1) keys.push_back({(uint32_t)de[c], {per * kss[i], 0, 0}});
            if (per > 1) inner.push_back({(uint32_t)per, {kss[i], 0, 0}});
            if (bs > 1) inner.push_back({(uint32_t)bs, {bss[i], 0, 0}});
        } else {
            return false;
        }
    }
    std::vector<SubDim> subs(keys);
    subs.insert(subs.end(), inner.begin(), inner.end());
    merged.clear();
    for (const SubDim &sd : subs) {
        if (!merged.empty() && merged.back().st[0] == (int64_t)sd.ext * sd.st[0] &&
            (uint64_t)merged.back().ext * sd.ext < (1ull << 31)) {
            merged.back().ext *= sd.ext;
            merged.back().st[0] = sd.st[0];
        } else {
            merged.push_back(sd);
        }
    }
    return true;
}

// Elements per access unit (up to 16 bytes): `vec` consecutive enumerated
// elements are one aligned vector on the other side when the fastest digit
// has stride 1 there and every stride keeps alignment.
static int rep_vec(const std::vector<SubDim> &merged, int64_t n, int esz)
{
    int vec = 16 / esz;
    auto ok = [&](int v) {
        if (merged.empty()) return n % v == 0;
        if (merged.back().st[0] != 1 || merged.back().ext % v) return false;
        for (const SubDim &sd : merged)
            if (&sd != &merged.back() && sd.st[0] % v) return false;
        return true;
    };
    while (vec > 1 && !ok(vec)) vec /= 2;
    return vec;
}

// Scatter (read the source in order, write the destination in runs) or gather
// (write the destination in order, read the source in runs).  Measured on
// MI355X for a 512 MiB fp32 re-blocking whose runs are 2 KiB either way
// (1024 x 2048 blocks to 4096 x 512): the scatter form 179-182 us against
// 185 us, as fast as a plain copy of the same bytes.  Tensors of 64 MiB and
// more take it when its access unit is no narrower; smaller ones, which their
// consumer usually reads next from the caches, keep the gather form.
static bool rep_prefer_scatter(int vg, int vs, int64_t bytes)
{
#ifdef TRA_REP_FORCE_SCATTER
    (void)vg; (void)vs; (void)bytes;
    return true;
#else
    return bytes >= (64ll << 20) && vs >= vg;
#endif
}

int tra_repartition(const int64_t *bounds, int rank, const int32_t *d_from, const int32_t *d_to, int dtype,
                    const void *src, void *dst, void *stream)
{
    if (!bounds || !d_from || !d_to) return fail(TRA_E_NULL, "NULL argument");
    if (rank < 1 || rank > kMaxRank) return fail(TRA_E_DLEN, "rank must be 1..12");
    if (dtype < D_F32 || dtype > D_I32) return fail(TRA_E_DTYPE, "unknown dtype");
    for (int i = 0; i < rank; ++i) {
        if (bounds[i] < 0) return fail(TRA_E_INDIVISIBLE, "extent < 0");
        if (bounds[i] == 0) {   // an empty tensor: nothing to move
            for (int j = 0; j < rank; ++j)
                if (d_from[j] < 1 || d_to[j] < 1 || (bounds[j] == 0 && (d_from[j] != 1 || d_to[j] != 1)) ||
                    (bounds[j] > 0 && (bounds[j] % d_from[j] || bounds[j] % d_to[j])))
                    return fail(TRA_E_INDIVISIBLE, "part count does not divide extent of dim " + std::to_string(j));
            return TRA_OK;
        }
    }
    if (!src || !dst) return fail(TRA_E_NULL, "NULL argument");
    if (!aligned16(src) || !aligned16(dst)) return fail(TRA_E_ALIGN, "device pointers must be 16-byte aligned");
    // label i of the tensor is the letter 'a' + i
    int64_t B[128] = {0};
    int32_t Du[128] = {0}, Dv[128] = {0};
    std::string t;
    int64_t n = 1;
    for (int i = 0; i < rank; ++i) {
        int c = 'a' + i;
        t.push_back((char)c);
        if (bounds[i] < 1) return fail(TRA_E_INDIVISIBLE, "extent < 1");
        if (d_from[i] < 1 || d_to[i] < 1 || bounds[i] % d_from[i] || bounds[i] % d_to[i])
            return fail(TRA_E_INDIVISIBLE, "part count does not divide extent of dim " + std::to_string(i));
        B[c] = bounds[i];
        Du[c] = d_from[i];
        Dv[c] = d_to[i];
        n *= bounds[i];
    }
    if (n >= (int64_t)1 << 31) return fail(TRA_E_RANGE, "tensor has 2^31 or more elements");
    RepartDesc r{};
    r.n_elems = n;
    const int esz = dtype_size(dtype);
    // Gather form: the destination is enumerated and read from the source.
    // Scatter form: the source is enumerated and written to the destination.
    std::vector<SubDim> gather, scatter;
    if (!rep_subdims(t, B, Du, Dv, gather) || !rep_subdims(t, B, Dv, Du, scatter))
        return fail(TRA_E_INDIVISIBLE, "in every dimension one block extent must divide the other");
    if (max_offset({{&gather, 0}}) >= n || max_offset({{&scatter, 0}}) >= n)
        return fail(TRA_E_RANGE, "internal: descriptor exceeds the tensor");
    const int vg = rep_vec(gather, n, esz), vs = rep_vec(scatter, n, esz);
    r.scatter = rep_prefer_scatter(vg, vs, n * esz);
    r.dst = to_radix(r.scatter ? scatter : gather);
    r.vec = r.scatter ? vs : vg;
    int err = launch_repartition(r, esz, src, dst, stream);
    if (err) return fail(TRA_E_HIP, std::string("kernel launch failed: ") + hip_error_text(err));
    return TRA_OK;
}

}  // extern "C"
