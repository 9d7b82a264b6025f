// graph.h -- EinGraph description, parsing and the partition-vector DP
// (internal; shared by the chooser and the graph executor).
#pragma once
#include <string>
#include <vector>

#include "plan.h"

namespace tra {

struct Cand {
    std::vector<int32_t> d;  // canonical order
    int64_t n_tasks = 0;
    int64_t cost = 0;        // node cost
    int64_t mem = 0;         // workspace bytes of its own step that depend on d (scratch, input copies)
    int64_t dp = 0;          // accumulated
    bool feasible = true;    // false: every way to feed it breaks the memory cap
    std::vector<int> pick;   // chosen producer candidate per input slot (-1 = graph input)
};

struct GNode {
    std::string name, kind, spec;
    std::vector<std::string> ops;
    std::string out, canon, con;
    int64_t B[128];
    std::vector<std::string> inputs;
    std::vector<int> src;    // producer node index per slot, -1 = graph input
    std::vector<Cand> cands;
    int in_dtype = D_BF16, out_dtype = D_F32;
    float scale = 1.0f;
};

// Parse the node-per-line description (see tra_choose in tra.h).
int parse_graph(const char *desc, std::vector<GNode> &nodes);

// Cost models of the chooser: the pages' numbers-moved model (admissible d:
// N >= P and N % P == 0), or the measured one-GPU time model (nanoseconds;
// every power-of-two d is a candidate, graph inputs arrive dense and the
// output is returned dense, so blockings other than all-ones on either
// cost a repartition).
enum CostModel { COST_PAGES = 0, COST_TIME = 1 };

// Choose d for every node (canonical label order per node) and the total cost.
// mem_cap > 0: the workspace live at every node's step (outputs still to be
// read, the node's repartition copies, its scratch) must fit in mem_cap bytes;
// candidates and producer choices that break it are pruned.  Results are
// memoised per (graph, P, model, cap).
int run_dp(std::vector<GNode> &nodes, int P, std::vector<std::vector<int32_t>> &d_out, int64_t &cost,
           int model = COST_PAGES, int64_t mem_cap = 0);

// Workspace bytes of one buffer as the graph executor lays it out.
inline int64_t ws_round(int64_t bytes) { return (bytes + 255) & ~(int64_t)255; }

// Measured time model (timemodel.cpp).
int64_t predict_plan_ns(const tra_plan_s &p);
int64_t predict_repartition_ns(int64_t elems, int dtype);

// The softmax node in one pass (k_simple.hip): true when the node's
// logsumexp plan `lse` and normalising plan `norm` can run as one kernel that
// holds each row in registers; the launcher writes the logsumexp and the
// normalised values.  Returns a hipError_t value.
bool softmax_one_pass(const tra_plan_s &lse, const tra_plan_s &norm);
int launch_softmax_rows(const tra_plan_s &lse, const tra_plan_s &norm, const void *s, void *lse_out, void *out,
                        void *stream);
int64_t predict_softmax_one_pass_ns(const tra_plan_s &lse, const tra_plan_s &norm);

// Two elementwise plans as one pass (k_simple.hip, tra_execute_chain): true
// when plan b's second operand is plan a's output in plan b's output layout.
bool elemwise_chainable(const tra_plan_s &a, const tra_plan_s &b);
// A matrix-core product followed by two elementwise steps in its epilogue:
//     t = join_a(product, ya) * scale_a       (rounded to the chain's dtype)
//     z = join_b(xb, t) * scale_b
// xb and z are laid out as the product's output; ya's offset is the sum of
// the st[0] strides of rb, rm and rn over the product's batch, row and column
// digits (the digits of the plan's gb, gm and gn).
struct ChainEpi {
    Pow2Group rb, rm, rn;
    const void *ya, *xb;
    int join_a, join_b;
    float scale_a, scale_b;
};
// The intermediate and output dtypes are equal (bf16, or fp32 when out_f32).
int launch_mfma_chain(const tra_plan_s &p, const ChainEpi &ce, bool out_f32, const void *x, const void *y, void *z,
                      void *stream);

int launch_elemwise_chain(const tra_plan_s &a, const tra_plan_s &b, const void *xa, const void *ya, const void *xb,
                          void *z, void *stream);

// Streams and events for the overlapped graph executor (streams.hip).  Return a
// hipError_t value (0 = success).
int current_device(int *dev);
int side_stream(void **out);
int events_create(int n, void **ev);
void events_destroy(int n, void **ev);
int event_record(void *ev, void *stream);
int stream_wait_event(void *stream, void *ev);

}  // namespace tra
