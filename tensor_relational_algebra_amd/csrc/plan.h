// plan.h -- host-side plan object and launcher interface (internal).
#pragma once
#include <string>

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
};

namespace tra {

// Launchers (kernels.hip).  Return a hipError_t value (0 = success).
int launch_generic(const tra_plan_s &p, const void *x, const void *y, void *z, void *stream);
int launch_elemwise(const tra_plan_s &p, const void *x, const void *y, void *z, void *stream);
int launch_rowreduce(const tra_plan_s &p, const void *x, const void *y, void *z, void *stream);
int launch_valu_tile(const tra_plan_s &p, const void *x, const void *y, void *z, void *ws, void *stream);
int launch_mfma_bf16(const tra_plan_s &p, const void *x, const void *y, void *z, void *ws, void *stream);
int launch_repartition(const RepartDesc &r, int elem_bytes, const void *src, void *dst, void *stream);
const char *hip_error_text(int err);

// Tile shapes the tile kernels are instantiated for.
struct TileShape { int bm, bn, bk; };
TileShape valu_tile_shape(int variant);
TileShape mfma_tile_shape(int variant);

void set_error(const std::string &msg);

}  // namespace tra
