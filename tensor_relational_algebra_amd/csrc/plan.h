// plan.h -- host-side plan object and launcher interface (internal).
#pragma once
#include <string>
#include <vector>

#include "tra.h"
#include "tra_internal.h"

struct tra_plan_s {
    std::string spec;
    int n_ops = 0;
    std::string xl, yl, zl, canon, con;
    int64_t B[128] = {0};
    int32_t d[128] = {0};
    int join = 0, agg = 0, in_dtype = 0, out_dtype = 0;
    float post_scale = 1.0f;
    tra_plan_info_t info{};
    int kernel = TRA_KERNEL_GENERIC;
    // lowering details
    tra::GenericDesc gen{};
    tra::GemmView gv{};
    tra::RowDesc row{};
    tra::ElemDesc el{};
    int tile = 0;              // tile-kernel variant index
    bool a_kmajor = true;      // X contiguous along K (else along M)
    bool b_kmajor = true;      // Y contiguous along K (else along N)
    bool ragged = false;       // vector-ALU tiles with masked edges (rag below)
    tra::RaggedMN rag{};
};

namespace tra {

// Launchers (kernels.hip).  Return a hipError_t value (0 = success).
int launch_generic(const tra_plan_s &p, const void *x, const void *y, void *z, void *ws, void *stream);
int launch_elemwise(const tra_plan_s &p, const void *x, const void *y, void *z, void *stream);
int launch_rowreduce(const tra_plan_s &p, const void *x, const void *y, void *z, void *ws, void *stream);
int launch_valu_tile(const tra_plan_s &p, const void *x, const void *y, void *z, void *ws, void *stream);
int launch_mfma_bf16(const tra_plan_s &p, const void *x, const void *y, void *z, void *ws, void *stream);
int launch_repartition(const RepartDesc &r, int elem_bytes, const void *src, void *dst, void *stream);
const char *hip_error_text(int err);

// Workspace of an int32 max-plus / min-plus tile plan: the split partials (if
// any), then the range-check flag words at this byte offset.
inline size_t small_int_flags_offset(int split, int64_t z_elems)
{
    return split > 1 ? ((size_t)split * (size_t)z_elems * 4 + 255) / 256 * 256 : 0;
}
constexpr size_t SMALL_INT_FLAG_BYTES = 256 * 4;

// Tile shapes the tile kernels are instantiated for.
struct TileShape { int bm, bn, bk; };
TileShape valu_tile_shape(int variant);
TileShape mfma_tile_shape(int variant);

void set_error(const std::string &msg);

// Relation-layout strides of a tensor with labels `t` (per label: in-block
// stride bs, key stride ks); B and d are indexed by label character.
void relation_strides(const std::string &t, const int64_t *B, const int32_t *d, int64_t *bs, int64_t *ks);

// One sub-dimension of a label group: extent and its stride in up to three tensors.
struct SubDim {
    uint32_t ext;
    int64_t st[3];
};
// Power-of-two digit group from sub-dimensions (most significant first);
// false if an extent is not a power of two or there are too many digits.
bool to_pow2(const std::vector<SubDim> &v, Pow2Group &g);

// Fused attention chain (scores join, softmax over keys, weighted-sum join).
int launch_attention(const AttnDesc &a, int out_dtype, const void *q, const void *k, const void *v, void *o,
                     void *stream);

}  // namespace tra
