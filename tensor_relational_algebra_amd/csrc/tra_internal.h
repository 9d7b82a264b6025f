// tra_internal.h -- descriptors passed from the host planner to the kernels.
//
// A relation (page "EinDecomp：基于爱因斯坦求和与张量关系代数的自动张量并行分解算法",
// section 2.2) is addressed through "sub-dimensions": every label l with part
// count d_l and block extent b_l contributes a key sub-dimension (extent d_l)
// and an in-block sub-dimension (extent b_l); the element offset in a tensor
// is the sum over its sub-dimensions of index * stride.  Sub-dimensions of
// extent 1 are dropped.  A flattened index over a list of sub-dimensions is
// mixed-radix with the last sub-dimension fastest.
#pragma once
#include <stdint.h>

namespace tra {

constexpr int kMaxLabels = 24;
constexpr int kMaxRank = 12;
constexpr int kMaxSub = 2 * kMaxRank;   // sub-dimensions of one index group

// Mixed-radix index space with runtime extents; strides into up to three
// tensors (0 = the tensor does not carry that sub-dimension).
struct Radix {
    int32_t n;
    uint32_t ext[kMaxSub];
    int64_t st[3][kMaxSub];
};

// Power-of-two index group: offset_t(idx) = sum_i ((idx >> sh_i) & mask_i) * st[t][i].
// At most kP2Max digits; unused digits have mask 0 (they add nothing), so the
// kernels evaluate all kP2Max digits unrolled, with every field in registers.
constexpr int kP2Max = 8;
struct Pow2Group {
    int32_t n;
    uint32_t total;
    uint32_t sh[kP2Max];
    uint32_t mask[kP2Max];
    int32_t st[3][kP2Max];
};

// Fused attention: digit groups of the query rows (s), key rows (t), heads
// (h) and head dimension (d) over the tensors that carry them.  Tensor slots:
// gs {Q, O}; gt {K, V}; gh {Q, K, V}; gho {O}; gd {Q, K, V}; gdo {O}.
struct AttnDesc {
    Pow2Group gs, gt, gh, gho, gd, gdo;
    uint32_t S, T, H, D;
    float scale_log2;   // scores scale times log2(e)
    int32_t o_vec4;     // O's four consecutive d are contiguous (vector stores)
};

// Join / aggregate codes (mirror tra.h).
enum Join : int32_t { J_MUL = 0, J_SQDIFF = 1, J_ADD = 2, J_IDENT = 3, J_EXP_SUB = 4, J_SUB = 5 };
enum Agg : int32_t { A_NONE = 0, A_SUM = 1, A_MAX = 2, A_MIN = 3, A_LSE = 4 };
enum DType : int32_t { D_F32 = 0, D_BF16 = 1, D_I32 = 2 };

// One-thread-per-output kernel: output positions enumerated in the output
// relation's own layout (so thread o writes z[o]); `out` gives X/Y strides of
// the output sub-dimensions (st[0] = X, st[1] = Y); `con` enumerates the
// contracted sub-dimensions, keys first (ascending key order), then in-block.
struct GenericDesc {
    Radix out;
    Radix con;
    int64_t n_out;
    int64_t n_con;
    float post_scale;
    // split > 0: few outputs over a long contracted range run as workgroups
    // of (chunk s, output o), each folding `chunk` consecutive contracted
    // indices with its four waves; split > 1 adds the in-order fold of the
    // chunks' partials (workspace [split][n_out])
    int32_t split;
    int64_t chunk;
};

// GEMM view of a two-operand EinSum: output labels only in X form M, only in
// Y form N, in both form B (batch); contracted labels (in both) form K.
// Group strides: gm {X, Z}, gn {Y, Z}, gk {X, Y}, gb {X, Y, Z}.
struct GemmView {
    Pow2Group gm, gn, gk, gb;
    int32_t split;          // workgroups sharing one output tile along K
    int32_t k_per_split;    // K extent each of them folds
    int64_t z_elems;        // for the split workspace stride
    float post_scale;
    int32_t z_vec4;         // four consecutive columns (from a multiple of 4) are contiguous in Z,
                            // and every other Z stride is a multiple of 4 elements
};

// Output row / column groups of a tile plan whose extents no tile divides or
// whose sub-dimensions are not all powers of two (vector-ALU tile kernel
// only): mixed-radix digits with strides {X, Z} for m and {Y, Z} for n, and
// the true extents; the GemmView's gm / gn then carry only the padded totals.
struct RaggedMN {
    Radix m, n;
    uint32_t M, N;
};

// Row reduction: one wavefront per output element; `out` as in GenericDesc;
// `outer` = contracted sub-dims except the last, `inner` = extent and X/Y
// strides of the last contracted sub-dim (X stride 1).
struct RowDesc {
    Radix out;
    Radix outer;
    int64_t n_out;
    int64_t n_outer;
    int64_t inner;
    int64_t inner_sy;
    float post_scale;
    // power-of-two form (p2 != 0): out_p2 / outer_p2 with st[0] = X, st[1] = Y;
    // inner is a multiple of 256 and inner_sy is 0 or 1
    int32_t p2;
    Pow2Group out_p2, outer_p2;
};

// Elementwise (aggregate NONE): `out` as in GenericDesc; vec elements of the
// fastest output sub-dimension are handled together when its X/Y strides
// allow (vx / vy: 1 = contiguous, 0 = broadcast, else scalar path).
struct ElemDesc {
    Radix out;
    int64_t n_out;
    int32_t vec;
    float post_scale;
    // power-of-two form (p2 != 0): out_p2 with st[0] = X, st[1] = Y; groups of
    // 4 outputs share one decomposition, X stride 1 along them, Y stride y_step (0 or 1)
    int32_t p2;
    int32_t y_step;
    Pow2Group out_p2;
};

// Repartition: destination positions enumerated in the destination layout;
// `dst` has, per destination sub-dimension, the source stride (st[0]).
// Runs of `vec` consecutive elements are contiguous in both layouts.
// A re-blocking copy.  Gather form (scatter == 0): unit u of the destination,
// in its own order, is read from the source offset that `dst` maps u to.
// Scatter form (scatter == 1): unit u of the source, in its own order, is
// written to the destination offset that `dst` maps u to.
struct RepartDesc {
    Radix dst;
    int64_t n_elems;
    int32_t vec;
    int32_t scatter;
};

}  // namespace tra
