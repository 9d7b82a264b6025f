/*
 * tra.h -- C ABI of libtra: extended EinSum executed as tensor-relational
 * algebra (TRA) join + aggregation on one AMD Instinct MI355X (gfx950).
 *
 * Method: page "EinDecomp：基于爱因斯坦求和与张量关系代数的自动张量并行分解算法"
 * (an EinDecomp summary).  Section 2.1 defines the extended EinSum (any
 * associative-commutative aggregate, any binary scalar join); section 2.2
 * defines tensor relations, the partition rule, and the three TRA operations
 * (join, aggregation, repartition) and the mechanical EinSum -> TRA lowering
 * under a partition vector d; sections 3.1-3.2 give the communication cost
 * model and the dynamic programme that choose d; section 4.3 prunes d to
 * powers of two and asks for task counts that are multiples of P.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every function returns a tra_status: 0 (TRA_OK) or a negative code.
 *   tra_last_error() gives a thread-local text for the last failure.  No C++
 *   exception crosses this boundary.
 * - All validation happens on the host before anything is launched; an
 *   error return means nothing was enqueued.
 * - Device pointers are plain HIP device addresses owned by the caller
 *   (libtra never allocates device memory; the only device resources it
 *   creates are, for TRA_GRAPH_OVERLAP_COPIES, one side stream per device and
 *   a graph's events).  Streams are hipStream_t passed as void*; NULL means
 *   the legacy default stream.  Calls are asynchronous with respect to the
 *   host: nothing synchronises.
 * - A "relation" is a tensor stored in the relation layout: given the
 *   tensor's labels l_1..l_n, extents B_l and part counts d_l (d_l | B_l,
 *   block extent b_l = B_l / d_l), the element with global index g sits at
 *       offset = rowmajor(k; d) * prod(b) + rowmajor(r; b),
 *       k_l = g_l / b_l,  r_l = g_l % b_l,
 *   i.e. the sub-tensors (section 2.2's partition rule) one after another in
 *   row-major key order, each sub-tensor dense row-major.  With every d_l = 1
 *   this is the ordinary dense row-major array.
 * - Canonical label order: the output labels in output order, then the
 *   contracted labels in order of first appearance (first operand, then the
 *   second).  bounds[] and d[] arguments follow it.
 * - Element counts of every tensor must stay below 2^31.
 * - Integer arithmetic is 32-bit two's complement (wrap-around), so integer
 *   results do not depend on the order of aggregation.
 */
#ifndef TRA_H
#define TRA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TRA_OK = 0,
    TRA_E_NULL = -1,          /* a required pointer argument is NULL */
    TRA_E_SPEC = -2,          /* spec string does not parse ("ab,bc->ac", "abc->ab") */
    TRA_E_LABELS = -3,        /* output label in no operand, label repeated in one operand,
                                 more than 24 labels, or rank above 12 */
    TRA_E_INDIVISIBLE = -4,   /* an extent < 1, a part count < 1, or d_l does not divide B_l */
    TRA_E_DLEN = -5,          /* n_labels differs from the spec's distinct label count, or a
                                 per-operand d vector has the wrong length / unequal shared entries */
    TRA_E_DTYPE = -6,         /* unknown dtype, or a dtype the op is not defined for
                                 (lse / exp_sub on integers, integer output of a float op) */
    TRA_E_OP = -7,            /* unknown join/aggregate, aggregate NONE with contracted labels,
                                 a binary join with one operand, ident with two, post_scale != 1
                                 on integers */
    TRA_E_WORKSPACE = -8,     /* workspace smaller than tra_plan_info().workspace_bytes */
    TRA_E_ALIGN = -9,         /* a device pointer is not 16-byte aligned */
    TRA_E_HIP = -10,          /* the HIP runtime reported an error at launch */
    TRA_E_NO_CANDIDATE = -11, /* the chooser found no admissible partition vector */
    TRA_E_RANGE = -12,        /* a tensor has 2^31 or more elements */
    TRA_E_GRAPH = -13,        /* malformed EinGraph description */
    TRA_E_BUFFER = -14        /* caller's output buffer too small */
} tra_status;

typedef enum { TRA_F32 = 0, TRA_BF16 = 1, TRA_I32 = 2 } tra_dtype;

/* Joins (section 2.1: any binary scalar function). */
typedef enum {
    TRA_JOIN_MUL = 0,     /* x * y */
    TRA_JOIN_SQDIFF = 1,  /* (x - y)^2 */
    TRA_JOIN_ADD = 2,     /* x + y */
    TRA_JOIN_IDENT = 3,   /* x (one operand) */
    TRA_JOIN_EXP_SUB = 4, /* exp(x - y) (float only) */
    TRA_JOIN_SUB = 5      /* x - y (integers wrap) */
} tra_join_op;

/* Aggregates (section 2.1: any associative and commutative reduction). */
typedef enum {
    TRA_AGG_NONE = 0,     /* no contracted label: Z = JOIN(...) */
    TRA_AGG_SUM = 1,
    TRA_AGG_MAX = 2,
    TRA_AGG_MIN = 3,
    TRA_AGG_LSE = 4       /* log(sum(exp(v))) (float only) */
} tra_agg_op;

/* Kernel family a plan was lowered to (reported by tra_plan_info). */
typedef enum {
    TRA_KERNEL_GENERIC = 0,   /* one thread per output element, any spec / op / layout */
    TRA_KERNEL_ELEMWISE = 1,  /* aggregate NONE, vectorised along the output's last label */
    TRA_KERNEL_ROWREDUCE = 2, /* one wavefront per output element, contiguous contracted run */
    TRA_KERNEL_VALU_TILE = 3, /* register-blocked output tiles on the vector ALUs */
    TRA_KERNEL_MFMA_BF16 = 4, /* bf16 x bf16 -> fp32 matrix-core tiles (mul + sum only) */
    TRA_KERNEL_EMPTY = 5      /* the output has no elements: nothing is enqueued */
} tra_kernel_family;

typedef struct tra_plan_s *tra_plan_t;

typedef struct {
    int64_t n_tasks;          /* N: join tasks = product of d over all labels */
    int64_t n_groups;         /* G: aggregation groups = product of d over the output labels */
    int64_t n_agg;            /* partials per group = product of d over contracted labels */
    int64_t agg_split;        /* workgroups that share one output tile (1 = in-register fold) */
    int64_t x_elems, y_elems, z_elems;
    size_t x_bytes, y_bytes, z_bytes;
    size_t workspace_bytes;   /* device scratch tra_execute needs (0 = none) */
    int32_t kernel;           /* tra_kernel_family */
    int32_t n_labels;
    char labels[32];          /* canonical label order, NUL-terminated */
    int32_t tile;             /* tile-kernel variant (mfma: 4 = 256x256 on four waves with 64-deep
                                 stages, for operands with runs of 8 or more elements along the
                                 dimension they are staged by; 5 = the same stages on a 256x128
                                 tile, for 128-wide outputs; 3 = 256x256 on four waves with 32-deep
                                 stages, 0 = 256x256 on eight waves, 1 = 128x128, 2 = 64x64;
                                 valu_tile: 1 = int32 max-plus / min-plus with the packed 16-bit
                                 path, see tra_execute, else 0); -1 if none */
} tra_plan_info_t;

/*
 * tra_plan -- lower one extended EinSum under a partition vector to a TRA
 * plan (section 2.2, "EinSum to TRA": partition X and Y by d, join every
 * key-matched sub-tensor pair, aggregate by the output part of the key;
 * section 3.1: a task is the triple (bound, EinSum, inputs)).
 *
 *   spec       "xlabels,ylabels->zlabels" or "xlabels->zlabels"; labels are
 *              single ASCII letters; at most 24 distinct labels, rank <= 12.
 *   bounds     n_labels extents B_l >= 0 in canonical label order.
 *   d          n_labels part counts d_l in canonical order, d_l | B_l (a zero
 *              extent takes d_l = 1).  The ≥P-tasks rule belongs to the
 *              chooser, not here: any d is run.
 *   join_op    tra_join_op; agg_op: tra_agg_op.
 *   in_dtype   dtype of both operands; out_dtype: dtype of Z.  Float
 *              inputs accumulate in fp32, integers in int32.
 *   post_scale multiplies the aggregated value (float only; 1 otherwise).
 *   out_plan   receives a host-only handle (no device work, no HIP call).
 * Empty tensors: an output with no elements plans to TRA_KERNEL_EMPTY (the
 * execution enqueues nothing); an empty contracted range (an operand with no
 * elements, the output not empty) makes every output element post_scale
 * times the aggregate's identity: 0 for sum, -inf / +inf for float max /
 * min, INT32_MIN / INT32_MAX for int32 max / min, -inf for lse.
 * Errors: TRA_E_NULL, TRA_E_SPEC, TRA_E_LABELS, TRA_E_DLEN,
 * TRA_E_INDIVISIBLE, TRA_E_DTYPE, TRA_E_OP, TRA_E_RANGE.
 */
int tra_plan(const char *spec, const int64_t *bounds, const int32_t *d, int n_labels,
             int join_op, int agg_op, int in_dtype, int out_dtype, float post_scale,
             tra_plan_t *out_plan);

/* Sizes and the lowering decision of a plan.  Errors: TRA_E_NULL. */
int tra_plan_info(tra_plan_t plan, tra_plan_info_t *info);

/* Free a plan's host memory.  NULL is accepted. */
int tra_plan_destroy(tra_plan_t plan);

/*
 * tra_execute -- run the plan's join + aggregation on the GPU
 * (section 2.2: join of key-matched pairs, then GROUP BY the output key and
 * reduce).  Each output sub-tensor's partials are folded in ascending order
 * of the contracted part of the key; no atomics, so runs are bitwise
 * reproducible.
 *
 *   x_rel, y_rel   operand relations under the plan's d (y_rel NULL for a
 *                  one-operand spec), dtype in_dtype, 16-byte aligned.
 *                  The pointer of a tensor with no elements may be NULL.
 *   z_rel          output relation under the plan's d restricted to the
 *                  output labels; fully overwritten.  Must not alias inputs.
 *   workspace      device scratch of at least info.workspace_bytes (may be
 *                  NULL when that is 0); contents on entry are ignored.
 *   hip_stream     hipStream_t the kernels are enqueued on.
 * An int32 add join aggregated by max or min on the vector-ALU tile kernel
 * (info.tile == 1) first checks on the device whether every element of X
 * and Y lies in [-1024, 1024].  If so, the join runs on packed binary16
 * halves, which hold every such sum exactly, so the output is the int32
 * result bit for bit; otherwise the 32-bit kernel runs.  The check writes its
 * flags into the last 1024 bytes of the workspace (so such plans always need
 * one), and the choice is made on the device with no host synchronisation.
 * Errors: TRA_E_NULL, TRA_E_ALIGN, TRA_E_WORKSPACE, TRA_E_HIP.
 */
int tra_execute(tra_plan_t plan, const void *x_rel, const void *y_rel, void *z_rel,
                void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * tra_execute_static -- tra_execute with no workspace argument, for callers
 * that cannot allocate device memory (code under stream capture, serving
 * loops, harnesses that forbid allocation).  The plan's scratch (the partials
 * of a split aggregation, the range-check flags of the packed max-plus path)
 * lives in one fixed array per device, tra_static_scratch_bytes() long (16
 * MiB), which the library holds on every device it runs on until the process
 * ends; its device address is looked up once per device, with that device
 * current, on the first call there.  Nothing is allocated or freed.
 * Every call on a device shares that device's array and its contents are
 * ignored on entry (every scratch byte a call reads it has written first),
 * so calls that overlap on one device (two streams, two threads) race and
 * must be ordered by the caller.  Arguments, layouts and errors as for
 * tra_execute; a plan whose info.workspace_bytes exceeds the array returns
 * TRA_E_WORKSPACE (use tra_execute with a workspace), and a failed symbol
 * lookup TRA_E_HIP.
 */
int tra_execute_static(tra_plan_t plan, const void *x_rel, const void *y_rel, void *z_rel, void *hip_stream);

/* Size in bytes of the per-device scratch array of tra_execute_static. */
size_t tra_static_scratch_bytes(void);

/*
 * tra_execute_chain -- two elementwise EinSums (aggregate NONE, section 2.1's
 * joins) as one pass, the first one's output never written:
 *     t = plan_a(xa, ya)       (rounded to plan_a's output dtype)
 *     z = plan_b(xb, t)        (t is plan_b's second operand)
 * The result is bit-identical to tra_execute(plan_a, ...) into a buffer t
 * followed by tra_execute(plan_b, xb, t, z): the fusion of consecutive
 * operators into one that the EinDecomp page's closing remarks point to.
 *
 *   plan_a, plan_b  elementwise plans whose outputs are the same relation
 *                   (same labels in the same order, same extents and d);
 *                   plan_b's second operand has plan_b's output labels in
 *                   the output's order; float dtypes, plan_b's input dtype
 *                   equal to plan_a's output dtype.
 *   xa, ya          plan_a's operand relations (ya NULL for one operand).
 *   xb              plan_b's first operand relation.
 *   z               plan_b's output relation; fully overwritten.
 * Errors: TRA_E_NULL, TRA_E_OP (the plans do not chain), TRA_E_ALIGN,
 * TRA_E_HIP.
 */
int tra_execute_chain(tra_plan_t plan_a, tra_plan_t plan_b, const void *xa, const void *ya, const void *xb,
                      void *z, void *hip_stream);

/*
 * tra_execute_contract_chain -- a contraction on the matrix cores followed by
 * two elementwise EinSums, all in the contraction's epilogue, so neither the
 * product nor the intermediate is ever written:
 *     p = plan_c(xc, yc)        (fp32, as tra_execute would store it)
 *     t = plan_a(p, ya)         (rounded to plan_a's output dtype)
 *     z = plan_b(xb, t)
 * The result is bit-identical to the three plans run one after the other.
 * This is the fusion of consecutive operators into one that the EinDecomp
 * page's closing remarks point to; the attention backward uses it for the
 * softmax Jacobian (dScores = Attn * (dO.V^T - r)).
 *
 *   plan_c   a bf16 mul/sum plan on the matrix-core kernel (info.kernel
 *            TRA_KERNEL_MFMA_BF16) with info.agg_split 1 and an fp32 output.
 *   plan_a   elementwise, two operands: its first operand and its output are
 *            plan_c's output relation (same labels, order, extents and d);
 *            its second operand ya carries output labels only (any subset,
 *            e.g. a per-row vector); fp32 input.
 *   plan_b   elementwise, two operands: both operands and the output are
 *            that same relation; t is its second operand.
 *   plan_a's output dtype, plan_b's input and output dtypes: one dtype,
 *   bf16 or fp32.
 *   xc, yc   plan_c's operand relations; ya, xb the steps' other operands;
 *   z        plan_b's output relation, fully overwritten.
 * Errors: TRA_E_NULL, TRA_E_OP (the plans do not fit the description
 * above), TRA_E_ALIGN, TRA_E_HIP.
 */
int tra_execute_contract_chain(tra_plan_t plan_c, tra_plan_t plan_a, tra_plan_t plan_b, const void *xc,
                               const void *yc, const void *ya, const void *xb, void *z, void *hip_stream);

/*
 * tra_repartition -- re-cut one tensor from partition vector d_from to d_to
 * (section 2.2, repartition; the initial partition of section 4.1's runtime
 * is the case d_from = all ones).  A pure permutation of elements: every
 * element is read once and written once, bit-exact.
 *
 *   bounds   rank extents >= 0; d_from, d_to: rank part counts each (a
 *            zero extent takes 1).  A tensor with no elements moves
 *            nothing; src and dst may then be NULL.
 *   dtype    tra_dtype (only its size matters).
 *   src,dst  device relations, 16-byte aligned, non-overlapping.
 * Errors: TRA_E_NULL, TRA_E_DLEN (rank < 1 or > 12), TRA_E_INDIVISIBLE,
 * TRA_E_DTYPE, TRA_E_ALIGN, TRA_E_RANGE, TRA_E_HIP.
 */
int tra_repartition(const int64_t *bounds, int rank, const int32_t *d_from,
                    const int32_t *d_to, int dtype, const void *src, void *dst,
                    void *hip_stream);

/*
 * tra_canonical_labels -- write the canonical label order of a spec
 * (output labels, then contracted labels by first appearance) into out
 * (NUL-terminated).  Returns the label count (> 0) or a negative status
 * (TRA_E_NULL, TRA_E_SPEC, TRA_E_LABELS, TRA_E_BUFFER).
 */
int tra_canonical_labels(const char *spec, char *out, int out_cap);

/*
 * tra_d_from_operand_form -- convert a per-operand partition vector (one
 * entry per label occurrence, first operand's labels then the second's, as
 * in section 2.2's matmul example [d_i, d_j, d_j, d_k]) to the canonical
 * per-label vector.  Occurrences of one label must agree (section 2.2
 * requires the two j entries to be equal).
 *   d_ops   n_ops entries; d_out: receives n_labels entries.
 * Errors: TRA_E_NULL, TRA_E_SPEC, TRA_E_LABELS, TRA_E_DLEN.
 */
int tra_d_from_operand_form(const char *spec, const int32_t *d_ops, int n_ops,
                            int32_t *d_out, int d_out_cap);

/*
 * tra_cost -- the communication cost of one EinSum under d (section 3.1):
 * N*(|X sub-tensor| + |Y sub-tensor|) + (N/n_agg)*(n_agg-1)*|Z sub-tensor|,
 * in elements, N being the node's join-task count.
 * Errors: as tra_plan's validation of spec/bounds/d.
 */
int tra_cost(const char *spec, const int64_t *bounds, const int32_t *d, int n_labels,
             int64_t *cost_out);

/*
 * tra_choose -- pick a partition vector for every node of an EinGraph by
 * the dynamic programme of section 3.2 over the cost model of section 3.1.
 *
 * graph_desc: one node per line, fields separated by blanks:
 *     <name> <kind> <spec> <label=extent,...> <input,input>
 *   kind is "einsum" or "softmax" (softmax: spec "hst->hst", the pair
 *   LSE = lse over the last label and Attn = exp(S - LSE) under one d);
 *   an input names an earlier node or, prefixed by '@', a graph input.
 *   Blank lines and lines starting with '#' are ignored.
 * P: required task multiple (a candidate needs N >= P and N % P == 0).
 * Candidates: every d_l a power of two dividing B_l (section 4.3).
 * Repartition term: 0 when the producer's part counts on its output labels
 * equal the consumer's on the matching input labels, else the tensor size.
 * Ties: lower cost, then fewer tasks, then the lexicographically smaller d.
 *
 *   d_out      receives, node after node in description order, each node's
 *              d in its canonical label order (d_cap entries available).
 *   cost_out   receives the total graph cost (may be NULL).
 * Errors: TRA_E_NULL, TRA_E_GRAPH, TRA_E_SPEC, TRA_E_LABELS,
 * TRA_E_NO_CANDIDATE, TRA_E_BUFFER.
 */
int tra_choose(const char *graph_desc, int P, int32_t *d_out, int d_cap, int64_t *cost_out);

/*
 * tra_choose_ex -- tra_choose with option flags.
 *
 * TRA_CHOOSE_TIME: replace the numbers-moved cost model by a time model
 * measured on one MI355X (the calibration that the EinDecomp page's closing
 * remarks ask a deployment to make: measured kernel and copy costs, a
 * per-launch latency, task granularity).  On one GPU every kernel reads its
 * operands in place under any blocking, so a node costs its kernels'
 * predicted time (tra_predict_ns of its plan under that d: launches times
 * the launch latency plus the larger of join terms / the measured rate of
 * the kernel family and tile the planner picks, and bytes / the measured
 * bandwidth), and a blocking change costs a repartition
 * (tra_predict_repartition_ns).  Graph inputs arrive dense and the output is
 * returned dense, so a node that needs an input, or leaves its output, in a
 * blocking other than all-ones pays that repartition too.  Every
 * power-of-two d is a candidate (P must still be >= 1 but is not a
 * constraint: the planner fills the chip by tiling and splitting).  The DP,
 * its tie-break and the output are those of tra_choose; cost_out is in
 * nanoseconds.
 * Errors: those of tra_choose; TRA_E_OP for an unknown flag.
 */
#define TRA_CHOOSE_TIME 1
/*
 * mem_cap_bytes (0 = none): the memory-aware variant of the DP (the
 * EinDecomp page's closing remarks: count the memory of outputs and
 * intermediates, prune plans over the limit).  The graph executor's
 * workspace at a node's step holds every output produced so far that is
 * still to be read, the node's own output, its repartitioned input copies,
 * a softmax node's logsumexp and the node's scratch; candidates, and
 * producer choices that would need a copy, are pruned when that exceeds the
 * cap (the executor's layout reaches that bound up to first-fit
 * fragmentation).  TRA_E_NO_CANDIDATE when nothing fits; TRA_E_OP for a
 * negative cap.
 * Results are memoised per (graph, P, flags, cap) for the life of the
 * process (the page's "optimise offline, load online"): a repeated call, or
 * tra_graph_plan* of the same graph, skips the DP (tra_choose_cache_stats,
 * tra_choose_cache_clear).
 */
int tra_choose_ex(const char *graph_desc, int P, int flags, int64_t mem_cap_bytes, int32_t *d_out, int d_cap,
                  int64_t *cost_out);

/* Hits and misses of the DP memo since the process started or the last clear.
 * Either pointer may be NULL.  Never fails. */
int tra_choose_cache_stats(int64_t *hits, int64_t *misses);

/* Empty the DP memo and zero its counters.  Never fails. */
int tra_choose_cache_clear(void);

/*
 * tra_predict_ns -- the time model's prediction, in nanoseconds, for one
 * tra_execute of `plan` (see TRA_CHOOSE_TIME).  Errors: TRA_E_NULL.
 */
int tra_predict_ns(tra_plan_t plan, int64_t *ns_out);

/*
 * tra_predict_repartition_ns -- predicted time of one tra_repartition of a
 * tensor of extents bounds[0..rank) and `dtype` whose blocking changes.
 * Errors: TRA_E_NULL, TRA_E_LABELS (rank outside 0..12), TRA_E_DTYPE,
 * TRA_E_INDIVISIBLE (a negative extent).
 */
int tra_predict_repartition_ns(const int64_t *bounds, int rank, int dtype, int64_t *ns_out);

/*
 * EinGraph executor (section 2.1: an EinGraph is a DAG of EinSum nodes whose
 * edges are tensors; section 4.1: the compiled plan partitions the inputs,
 * runs every node's join + aggregation, and reorganises intermediates whose
 * producer and consumer blockings differ).
 *
 * tra_graph_plan -- parse a graph (the tra_choose line format; each line may
 * end with options in=<dtype> out=<dtype> scale=<float>: the dtype both
 * operands are stored in, the dtype of the node's output, and post_scale),
 * pick d for every node (d_all == NULL: the tra_choose DP with task multiple
 * P; else d_all holds every node's d in canonical order, concatenated, d_len
 * entries), plan every node, and lay out the device workspace the run needs.
 * A softmax node "hst->hst" is run as LSE[h,s] = lse_t S (ident + lse, fp32)
 * then Attn = exp(S - LSE) (exp_sub, aggregate NONE, written in out dtype),
 * both under the node's d.
 * Graph inputs ('@' names) are numbered in order of first appearance; each is
 * passed dense row-major, shaped as its consumer writes it, in the
 * consumer's in dtype.  The output node's result is returned dense row-major.
 * Errors: those of tra_choose and tra_plan.
 */
typedef struct tra_graph_s *tra_graph_t;

typedef struct {
    int32_t n_nodes;
    int32_t n_leaves;
    size_t workspace_bytes;   /* device scratch tra_graph_execute needs: buffers whose
                                 live steps overlap are disjoint, others share bytes */
    int64_t out_elems;        /* elements of the output node's result */
    int32_t out_dtype;
    int64_t cost;             /* cost-model value of the chosen partition vectors */
    int32_t n_repartitions;   /* inter-node repartitions the plan contains */
    int32_t n_fused;          /* attention chains run as one fused kernel */
} tra_graph_info_t;

int tra_graph_plan(const char *graph_desc, int P, const int32_t *d_all, int d_len, tra_graph_t *out_graph);

/*
 * tra_graph_plan_ex -- tra_graph_plan with option flags.
 *
 * TRA_GRAPH_FUSE_ATTENTION: every chain
 *     S = scale * sum_d Q[s,h,d] K[t,h,d]   (einsum, 2 inputs, bf16 operands)
 *     A = softmax over t of S              (softmax node on S, its only consumer)
 *     O = sum_t A[h,s,t] V[t,h,e]           (einsum, A as first input, its only consumer)
 * (labels named freely, in any order; one head label h, head dimension
 * d = e in {32, 64, 128}, S a multiple of 128 and T of 64, power-of-two
 * partition counts, Q/K/V contiguous along the head dimension) is run as one
 * kernel that folds the logsumexp over the t blocks online and never writes S
 * or A (the "super-operator" fusion that the EinDecomp page's closing remarks
 * point to).  Q, K and V are read in the blockings of their producers (no
 * repartition), O is written in the O node's blocking.  The score and softmax
 * nodes then enqueue nothing in tra_graph_run_node.  Chains that do not match
 * run unfused; tra_graph_info reports how many were fused.
 * The partition vectors are still chosen per node by the cost model.
 * Numerics: the probabilities enter the weighted sum as bf16 (the unfused
 * path also stores A in bf16), relative to the running maximum rather than
 * normalised; O is divided by the fp32 sum at the end.
 * Errors: those of tra_graph_plan; TRA_E_OP for an unknown flag.
 */
#define TRA_GRAPH_FUSE_ATTENTION 1
/*
 * TRA_GRAPH_CHOOSE_TIME: when d_all is NULL, choose the partition vectors
 * with the measured time model (TRA_CHOOSE_TIME) instead of the pages'
 * numbers-moved model; tra_graph_info's cost is then in nanoseconds.
 */
#define TRA_GRAPH_CHOOSE_TIME 2
/*
 * TRA_GRAPH_OVERLAP_COPIES: tra_graph_execute runs every repartition copy on
 * a second stream of the current device (created on first use, default
 * priority, kept for the life of the process) while the nodes run in order on
 * the caller's stream: a graph input's copy starts at once, an intermediate's
 * as soon as its producer has run, and each consumer waits for its copies
 * through events.  The workspace layout keeps each copy live from its
 * producer's step (a graph input's: from the start) to its consumer's, so it
 * can be larger than without the flag.  All work is joined back into the
 * caller's stream before the output node runs, so the call's completion is
 * still observed on that stream; calls on one graph object must not overlap
 * in time (they share its events).  tra_graph_run_node is unaffected.
 */
#define TRA_GRAPH_OVERLAP_COPIES 4
int tra_graph_plan_ex(const char *graph_desc, int P, const int32_t *d_all, int d_len, int flags,
                      tra_graph_t *out_graph);

/*
 * tra_graph_plan_cap -- tra_graph_plan_ex with the partition vectors chosen
 * under a workspace cap (see tra_choose_ex's mem_cap_bytes; 0 = none).
 * Errors: those of tra_graph_plan_ex; TRA_E_NO_CANDIDATE when nothing fits;
 * TRA_E_OP for a negative cap.
 */
int tra_graph_plan_cap(const char *graph_desc, int P, int flags, int64_t mem_cap_bytes, tra_graph_t *out_graph);

/* Sizes of a planned graph.  Errors: TRA_E_NULL. */
int tra_graph_info(tra_graph_t graph, tra_graph_info_t *info);

/* d of node `node` (canonical order) into d_out; returns its length or a
 * negative status (TRA_E_NULL, TRA_E_GRAPH for a bad index, TRA_E_BUFFER). */
int tra_graph_node_d(tra_graph_t graph, int node, int32_t *d_out, int d_cap);

/* Graph input `leaf`: NUL-terminated name (without '@') into name, element
 * count and dtype.  Errors: TRA_E_NULL, TRA_E_GRAPH, TRA_E_BUFFER. */
int tra_graph_leaf(tra_graph_t graph, int leaf, char *name, int name_cap, int64_t *elems, int32_t *dtype);

/*
 * tra_graph_node_output -- where node `node` leaves its output relation in the
 * workspace (EinDecomp page, section 2.2: every intermediate is a relation
 * blocked by its producer's d).  After tra_graph_run_node of that node, and
 * until a later node reuses those bytes (the workspace is laid out by
 * liveness), the relation is at byte `*offset` of the workspace: `*elems`
 * elements of `*dtype`, blocked by the node's d (tra_graph_node_d) restricted
 * to its output labels, in output-label order.  A softmax node also leaves its
 * logsumexp over the last label (fp32, blocked the same way over the other
 * labels, `*lse_elems` elements) at `*lse_offset`; for any other node
 * `*lse_elems` is 0 and `*lse_offset` SIZE_MAX.  Nothing is read or written
 * on the device.
 * Errors: TRA_E_NULL, TRA_E_GRAPH (bad index), TRA_E_OP for a node folded
 * into a fused attention chain (it writes no output of its own).
 */
int tra_graph_node_output(tra_graph_t graph, int node, size_t *offset, int64_t *elems, int32_t *dtype,
                          size_t *lse_offset, int64_t *lse_elems);

/*
 * tra_graph_run_node -- enqueue one node: the repartitions its inputs need
 * (graph inputs: dense -> the node's blocking; intermediates: only when the
 * producer's blocking differs), then its join + aggregation.  For the output
 * node, `out` (may be NULL otherwise) receives the dense result.  Nodes must
 * be run in description order.  leaves: n_leaves device pointers.
 * Errors: TRA_E_NULL, TRA_E_GRAPH, TRA_E_WORKSPACE, TRA_E_ALIGN, TRA_E_HIP.
 */
int tra_graph_run_node(tra_graph_t graph, int node, const void *const *leaves, int n_leaves, void *out,
                       void *workspace, size_t workspace_bytes, void *hip_stream);

/* Every node in order (tra_graph_run_node for each; with
 * TRA_GRAPH_OVERLAP_COPIES the copies run on a side stream, see above). */
int tra_graph_execute(tra_graph_t graph, const void *const *leaves, int n_leaves, void *out, void *workspace,
                      size_t workspace_bytes, void *hip_stream);

/* Free a graph's host memory.  NULL is accepted. */
int tra_graph_destroy(tra_graph_t graph);

/*
 * tra_probe_mfma_loop -- measurement aid: `workgroups` workgroups of four
 * waves each run `iters` rounds of 8 independent bf16 32x32x16 matrix-core
 * products on register operands (2 * 32 * 32 * 16 * 8 * 4 flop per round and
 * workgroup), the ceiling the tile kernels are held against beside the
 * published peak.  distinct_operands = 0: all 8 products take one operand
 * pair; otherwise each takes its own random values (of the size of the
 * products' N(0, 0.02) inputs), so the multipliers switch operands from one
 * product to the next as in a real product, and the chip's power limit sets
 * the clock as it does there.  distinct_operands = 2: rounds of 64 independent
 * 16x16x32 products (2 * 16 * 16 * 32 * 64 * 4 flop per round and workgroup)
 * on random operands, the product form of the 64-deep tile.  out: device
 * buffer of workgroups * 256 floats (written, values meaningless).  Errors:
 * TRA_E_NULL, TRA_E_OP (counts < 1), TRA_E_HIP.
 */
int tra_probe_mfma_loop(int workgroups, int iters, int distinct_operands, float *out, void *hip_stream);

/* Text of a status code (static storage). */
const char *tra_status_string(int status);

/* Thread-local detail of the last failure on this thread ("" if none). */
const char *tra_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* TRA_H */
