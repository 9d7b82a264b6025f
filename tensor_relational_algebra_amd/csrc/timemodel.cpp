// timemodel.cpp -- measured one-GPU time model for the chooser.
//
// The cost model of the page "EinDecomp：基于爱因斯坦求和与张量关系代数的自动张量
// 并行分解算法" (section 3.1) counts numbers moved between devices; its closing
// remarks list what a deployment should calibrate: the measured cost of
// each communication pattern and kernel, a per-launch latency, and a minimum
// task granularity.  On one MI355X the "devices" are workgroups and nothing
// crosses a network: a node's time is its kernel's time, which the kernels
// reach for any blocking because they read every operand in place, and a
// change of blocking between two nodes is a repartition copy through HBM.
// The model charges exactly that:
//
//   node(plan)        = launches * latency
//                       + max(terms / rate(kernel family, tile),
//                             bytes read and written once / bandwidth)
//                       (+ the cross-workgroup fold's bytes when split > 1)
//   repartition(T)    = latency + 2 * |T| * sizeof(dtype) / copy bandwidth
//
// terms = the number of join evaluations (the product of all label extents).
// The constants were measured on one MI355X by `bench.py --calibrate`
// (launch latency: a chain of one-wavefront EinSum nodes run by one
// tra_graph_execute; rates and bandwidths: each kernel family at a size that
// fills the chip).  Minimum granularity needs no term of its own:
// a plan whose output tiles cannot fill the chip is split over the
// contracted range by the planner, and the small-tile variants carry their
// own, lower, measured rates.
#include <algorithm>
#include <cmath>

#include "graph.h"

namespace tra {

// Calibration (MI355X, one GPU, measured by `bench.py --calibrate`).  Rates
// in join terms per nanosecond, bandwidths in bytes per nanosecond.
struct Calibration {
    double latency_ns = 3700.0;        // per node of back-to-back launches from the library
    // bf16 matrix cores, tile variants 0/1/2/3/4/5 (launch latency taken out;
    // the narrow 64-deep tile, 5, is priced as the 128 x 128 tile it replaces)
    double mfma_terms[6] = {487e3, 163e3, 90e3, 518e3, 518e3, 163e3};
    double valu_terms = 22.1e3;        // register-tiled vector-ALU joins (squared distance)
    double valu_small_int_terms = 35.0e3;   // int32 max / min-plus on packed 16-bit halves, range check included
                                            // (inputs within +-1024; outside, the 32-bit path runs at valu_terms)
    double rowreduce_terms = 1155.0;   // one wavefront per output element, compute-bound
    double generic_terms = 1046.0;     // one thread per output element
    double rowreduce_bw = 5025.0;      // row-reduce, bandwidth-bound (logsumexp over t)
    double stream_bw = 5520.0;         // elementwise and one-thread-per-output kernels
    double tile_bw = 6080.0;           // bandwidth bound of the tile kernels (small-tile matrix-core case)
    double copy_bw = 5755.0;           // repartition
    double softmax_bw = 5700.0;        // the softmax node in one pass (5511 and 5935 on the attention layer)
};
static const Calibration kCal;

static double dtype_bytes(int dt) { return dt == D_BF16 ? 2.0 : 4.0; }

int64_t predict_plan_ns(const tra_plan_s &p)
{
    const tra_plan_info_t &in = p.info;
    if (p.kernel == TRA_KERNEL_EMPTY) return 0;
    double terms = 1.0;
    for (char c : p.canon) terms *= (double)p.B[(int)c];
    const double bytes = (double)in.x_bytes + (double)in.y_bytes + (double)in.z_bytes;
    double rate;
    double bw = kCal.stream_bw;
    switch (p.kernel) {
    case TRA_KERNEL_MFMA_BF16:
        rate = kCal.mfma_terms[std::min(std::max(p.tile, 0), 5)];
        bw = kCal.tile_bw;
        break;
    case TRA_KERNEL_VALU_TILE:
        rate = p.tile == 1 ? kCal.valu_small_int_terms : kCal.valu_terms;
        bw = kCal.tile_bw;
        break;
    case TRA_KERNEL_GENERIC:
    case TRA_KERNEL_ROWREDUCE:
        if (p.gen.split > 0) {
            // few outputs, each folded by whole workgroups: bandwidth-bound
            rate = 1e30;
            bw = kCal.rowreduce_bw;
        } else if (p.kernel == TRA_KERNEL_GENERIC) {
            rate = kCal.generic_terms;
        } else {
            rate = kCal.rowreduce_terms;
            bw = kCal.rowreduce_bw;
        }
        break;
    default: rate = 1e30; break;   // elementwise: bandwidth-bound
    }
    double t = kCal.latency_ns + std::max(terms / rate, bytes / bw);
    if (in.agg_split > 1)
        t += kCal.latency_ns + (double)(in.agg_split + 1) * (double)in.z_elems * 4.0 / kCal.stream_bw;
    return (int64_t)std::llround(t);
}

// The softmax node as one pass: S read once, the output and the logsumexp
// written once.
int64_t predict_softmax_one_pass_ns(const tra_plan_s &lse, const tra_plan_s &norm)
{
    const double bytes = (double)lse.info.x_bytes + (double)norm.info.z_bytes + (double)lse.info.z_bytes;
    return (int64_t)std::llround(kCal.latency_ns + bytes / kCal.softmax_bw);
}

int64_t predict_repartition_ns(int64_t elems, int dtype)
{
    if (elems <= 0) return 0;
    return (int64_t)std::llround(kCal.latency_ns + 2.0 * (double)elems * dtype_bytes(dtype) / kCal.copy_bw);
}

}  // namespace tra

using namespace tra;

extern "C" int tra_predict_ns(tra_plan_t plan, int64_t *ns_out)
{
    if (!plan || !ns_out) {
        set_error("plan / ns_out is NULL");
        return TRA_E_NULL;
    }
    *ns_out = predict_plan_ns(*plan);
    return TRA_OK;
}

extern "C" int tra_predict_repartition_ns(const int64_t *bounds, int rank, int dtype, int64_t *ns_out)
{
    if (!bounds || !ns_out) {
        set_error("bounds / ns_out is NULL");
        return TRA_E_NULL;
    }
    if (rank < 0 || rank > 12) {
        set_error("rank out of range");
        return TRA_E_LABELS;
    }
    if (dtype < D_F32 || dtype > D_I32) {
        set_error("unknown dtype");
        return TRA_E_DTYPE;
    }
    int64_t n = 1;
    for (int i = 0; i < rank; ++i) {
        if (bounds[i] < 0) {
            set_error("negative extent");
            return TRA_E_INDIVISIBLE;
        }
        n *= bounds[i];
    }
    *ns_out = predict_repartition_ns(n, dtype);
    return TRA_OK;
}
