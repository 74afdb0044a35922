/*
 * dqg.h -- quantised GEMV and expert-MLP kernels for AMD Instinct MI355X
 * (gfx950), C ABI.
 *
 * The operations are the decode-time calls over resident quantised weights
 * that the API-contract section of "colibri Vulkan compute backend complete
 * guide" (xdnf.cn) lists:
 *   - a single quantised GEMV (its coli_vk_matmul);
 *   - the first half of an expert MLP, silu(gate(x)) * up(x), with x read
 *     once (its coli_vk_gate_up);
 *   - the whole fused MLP of a batch of routed experts, hidden state kept
 *     on the device, synchronous or issued and joined later (its
 *     coli_vk_expert_group, _issue and _take).
 *
 * Weight formats are the device formats of colibri's expert tier ("colibri
 * -- Vulkan backend (docs/vulkan.md)", expert-tier engine table; values and
 * packing from the shader-level section of the guide above):
 *   DQG_I8_ROW  (1)  int8, two's complement, one f32 scale per row
 *   DQG_I4_ROW  (2)  int4 pairs, value = nibble - 8, one f32 scale per row
 *   DQG_I4_GS   (4)  int4 pairs, value = nibble - 8, one f32 scale per gs inputs
 *   DQG_I3_G64  (5)  int3 in two bit planes, value = code - 4, one f32 scale per 64
 *   DQG_MXFP4   (7)  e2m1 nibbles, bit 3 the sign, one f32 scale per 32
 *                    (the e8m0 scale pre-expanded to f32 by the host)
 *   DQG_F32     (10) f32 rows, no scales
 *   DQG_BF16    (11) bf16 rows, no scales
 *   DQG_FP8_BLOCK (12) OCP FP8 E4M3 (no infinities, S.1111.111 NaN), one
 *                    f32 scale per block of 128 rows x 128 inputs
 *   DQG_I8_GS   (13) int8, two's complement, one f32 scale per gs inputs
 *   DQG_F16     (14) f16 rows, no scales
 * (formats 10 to 14: the same engine table, the qwen36 and qwen38 rows, and
 * the f16-rows paragraph of that page: no scales, the even column in the
 * low half of a word, as for bf16.)
 *
 * Storage of one matrix W with O rows of K inputs (all row-major):
 *   fmt 1:        q = int8 [O][K]                          scales = f32 [O]
 *   fmt 2, 4, 7:  q = uint8 [O][K/2]; byte j of a row holds input 2j in its
 *                 low nibble and input 2j+1 in its high nibble
 *                                                          scales = f32 [O][K/gs]
 *   fmt 5:        q  = uint32 [O][K/16]: 2 bits per input, input k at bits
 *                      2*(k mod 16) of word k/16;
 *                 q2 = uint32 [O][K/32]: 1 bit per input, input k at bit
 *                      (k mod 32) of word k/32;
 *                 code = low | high << 2               scales = f32 [O][K/64]
 *   fmt 10:       q = f32 [O][K]                           scales = NULL
 *   fmt 11, 14:   q = uint16 [O][K] (bf16 or f16 bits, little-endian, so
 *                 the even input is the low half of each 32-bit word)
 *                                                          scales = NULL
 *   fmt 12:       q = uint8 [O][K] (E4M3 bits)
 *                                          scales = f32 [ceil(O/128)][K/128]
 *                 (weight (o, k) takes scale [o/128][k/128])
 *   fmt 13:       q = int8 [O][K]                          scales = f32 [O][K/gs]
 * (The pages do not fix nibble order, plane bit order or the layout of the
 * FP8 block scales; these are the readings this library and its tests use.)
 *
 * A weight is value * scale.  y[s][o] = sum_k W[o][k] * x[s][k] in f32.
 * Results match a double-precision evaluation of that sum to within 1e-5
 * of sum_k |W[o][k] * x[s][k]| per row; dequantised weights match the
 * f32 rounding of value * scale bit for bit.
 *
 * Conventions for every call:
 *   - Every array argument is a DEVICE pointer owned by the caller; nothing
 *     is copied to or from the host.  The library owns only an expert
 *     table's device descriptor array.
 *   - Base pointers of q, q2, x, y, h and scratch must be 16-byte aligned;
 *     scales 4-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls enqueue
 *     kernels and return without synchronising the host, except
 *     dqg_expert_group_take, dqg_expert_table_create/destroy.
 *   - Arguments are validated before anything is enqueued.  On a non-zero
 *     return nothing was launched and no output was written; the reason is
 *     in dqg_last_error() (per thread).
 *   - Work on one stream is ordered as usual; calls on different streams
 *     that write the same buffers race.
 */
#ifndef DQG_H
#define DQG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DQG_OK = 0,
    DQG_EINVAL = -1,   /* NULL or misaligned pointer, bad count or option */
    DQG_EFORMAT = -2,  /* unknown format, or a group size the format does not have */
    DQG_ESHAPE = -3,   /* shapes that disagree or do not divide into whole groups */
    DQG_EDEVICE = -4,  /* a HIP runtime call failed */
    DQG_ELAUNCH = -5,  /* a kernel launch failed (or DQG_FAULT injected a failure) */
    DQG_ENOMEM = -6,   /* scratch too small, or a device allocation failed */
    DQG_EROUTE = -7    /* dqg_expert_group_take: an expert id was out of range */
} dqg_status;

enum {
    DQG_I8_ROW = 1,
    DQG_I4_ROW = 2,
    DQG_I4_GS = 4,
    DQG_I3_G64 = 5,
    DQG_MXFP4 = 7,
    DQG_F32 = 10,
    DQG_BF16 = 11,
    DQG_FP8_BLOCK = 12,
    DQG_I8_GS = 13,
    DQG_F16 = 14
};

/* One resident quantised matrix (device pointers, caller-owned).
 * gs: inputs per scale; K for fmt 1 and 2, a power of two >= 32 dividing K
 * for fmt 4 and 13, 64 for fmt 5, 32 for fmt 7, 128 for fmt 12, 0 or K for
 * the formats without scales (10, 11, 14), whose scales must be NULL.
 * K must be a multiple of 16 (fmt 1), 32 (fmt 2, 4, 7), 64 (fmt 5), 128
 * (fmt 12), 4 (fmt 10) or 8 (fmt 11, 14).  q2 is used by fmt 5 only. */
typedef struct {
    int32_t fmt;
    int32_t O;
    int32_t K;
    int32_t gs;
    const void *q;
    const void *q2;
    const float *scales;
} dqg_matrix;

/* One expert's three matrices: gate and up are [I x H], down is [H x I]. */
typedef struct {
    dqg_matrix gate;
    dqg_matrix up;
    dqg_matrix down;
} dqg_expert;

/* Byte offset of h inside an expert-group scratch buffer (see below). */
#define DQG_SCRATCH_H_OFFSET 1024

/* Opaque: a device copy of the experts' descriptors (owned by the library). */
typedef struct dqg_expert_table dqg_expert_table;

/* Handle of an issued expert-group call. */
typedef struct {
    void *event;          /* hipEvent_t recorded after the call's kernels */
    const int32_t *flag;  /* device word the kernels set when an id was out of range */
    int32_t status;       /* DQG_OK until dqg_expert_group_take reports otherwise */
} dqg_ticket;

/* Counters of calls, launches and host-known algorithmic bytes. */
typedef struct {
    uint64_t calls_matmul;
    uint64_t calls_gate_up;
    uint64_t calls_dequant;
    uint64_t calls_expert_group;
    uint64_t launches;
    uint64_t bytes;   /* weight codes + scales + x + y of matmul, gate_up, dequant */
    uint64_t calls_route;
} dqg_counters;

/*
 * y[s][o] = sum_k W[o][k] * x[s][k] for s < S.
 * Quantised GEMV (the guide's API-contract section, coli_vk_matmul; the
 * shader-level section for the decode).  x: f32 [S][K]; y: f32 [S][O].
 * S >= 1.  Two routes, each giving a token's row the same bits whatever S
 * is: up to 8 tokens the per-row route; from 9 tokens, for formats 1, 4, 7,
 * 12, 13 and 14 with K a multiple of 32, the matrix-core GEMM (the bits of
 * the two routes differ within the error bound).  When the GEMM's grid is
 * too small for the chip it splits K and keeps the partial sums in a device
 * buffer that the library allocates on first need (hipMalloc, one per
 * device, grown to at most 1 GiB, held until the process ends); calls on
 * different streams take turns with it, in the order they were made.  A
 * stream under graph capture uses no such buffer.
 */
int dqg_matmul(const dqg_matrix *W, const float *x, int32_t S, float *y, void *stream);

/*
 * h[s][i] = silu(G[i] . x[s]) * (U[i] . x[s]), silu(z) = z / (1 + e^-z).
 * The SwiGLU half of an expert MLP in one launch with x read once (the
 * guide's API-contract section, coli_vk_gate_up).  G and U: [I x H] of one
 * format; x: f32 [S][H]; h: f32 [S][I].  Routes and the partials buffer as
 * for dqg_matmul, with the GEMM from 8 tokens (9 for formats 1 and 13).
 */
int dqg_gate_up(const dqg_matrix *G, const dqg_matrix *U, const float *x, int32_t S, float *h,
                void *stream);

/*
 * dqg_gate_up with the clamped SwiGLU (swiglu_limit L):
 *   h = silu(min(G.x, L)) * min(max(U.x, -L), L).
 * ("colibri -- Vulkan backend (docs/vulkan.md)", the GLM paragraph: the
 * experts' SwiGLU is clamped; a limit of 0 zeroes every expert's output and
 * the backend's shader runs only above 0.)  L > 0, or +inf for the plain
 * SwiGLU (the same bits as dqg_gate_up); other values give DQG_EINVAL.  A
 * NaN in g or u stays NaN.  Everything else as dqg_gate_up.
 */
int dqg_gate_up_clamped(const dqg_matrix *G, const dqg_matrix *U, const float *x, int32_t S, float limit,
                        float *h, void *stream);

/*
 * out[o][k] = value(o, k) * scale(o, k), rounded once to f32.
 * Materialises the dequantised weights (for bit-exact checks of the decode
 * that the other calls do in registers).  out: f32 [O][K].
 */
int dqg_dequant(const dqg_matrix *W, float *out, void *stream);

/*
 * Build the device descriptor table of n_experts experts (all with the same
 * gate/up format, group size and [I x H] shape, and the same down format,
 * group size and [H x I] shape).  Synchronous (one small host-to-device
 * copy on the current device).  The pointed-to weights stay caller-owned
 * and must outlive the table.  The resident-expert table stands for the
 * device registry of the guide's "what runs on the GPU" section.
 */
int dqg_expert_table_create(const dqg_expert *experts, int32_t n_experts, dqg_expert_table **out);
void dqg_expert_table_destroy(dqg_expert_table *table);

/* The limit of the table's experts' SwiGLU in dqg_expert_group (the clamped
 * form of dqg_gate_up_clamped): L > 0, or +inf (the default at creation)
 * for the plain SwiGLU; other values give DQG_EINVAL and leave it as it
 * was.  Applies to calls issued after it returns. */
int dqg_expert_table_set_swiglu_limit(dqg_expert_table *table, float limit);

/*
 * The experts' activation in dqg_expert_group:
 *   DQG_ACT_SWIGLU (the default at creation): h = SwiGLU(g, u) with the
 *     table's limit; y[t] adds w[t][r] * down(h) in rank order, then the
 *     shared expert.
 *   DQG_ACT_SWIGLU_V4: DeepSeek V4's rounding form ("colibri -- Vulkan
 *     backend (docs/vulkan.md)", the paragraph on DeepSeek V4's CPU expert
 *     and the tier's third activation).  g and u are rounded to bf16 before
 *     the (clamped) SwiGLU; the activation times the slot's route weight
 *     (1 for the shared expert) is rounded to bf16; each block of 128
 *     consecutive values of a slot's h is rounded to E4M3 after division
 *     by the block's scale, the smallest power of two that takes the
 *     block's largest magnitude below 448, and multiplied back; down's
 *     output is rounded to bf16; y[t] is the f32 sum from 0 of the token's
 *     routed rows in ascending (expert id, rank), then the shared row, with
 *     no further weight.  Every rounding is to nearest, ties to even.  The
 *     scratch's h then holds down's input (the scaled E4M3 values).  x is
 *     used as given: the pages' engine rounds it to E4M3 per 128 on the host
 *     before the call.  Needs I to be a multiple of 128 (DQG_EINVAL
 *     otherwise); adds one launch ("group_act_v4") between gate/up and down.
 * Other values give DQG_EINVAL and leave the table as it was.  Applies to
 * calls issued after it returns.
 */
#define DQG_ACT_SWIGLU 0
#define DQG_ACT_SWIGLU_V4 1
int dqg_expert_table_set_activation(dqg_expert_table *table, int32_t act);

/* Scratch bytes dqg_expert_group needs for S tokens of top-k routing: a
 * header of DQG_SCRATCH_H_OFFSET bytes (the error flag at byte 0), then the
 * hidden state h of every (token, rank) and shared slot.  The scratch needs
 * no initialisation, and one scratch serves calls of any size up to the
 * one it was sized for (calls that share a scratch must not overlap). */
size_t dqg_expert_group_scratch_bytes(const dqg_expert_table *table, int32_t S, int32_t k);

/*
 * y[t] = sum_{r<k} w[t][r] * MLP_{ids[t][r]}(x[t]) + MLP_shared(x[t])
 * with MLP_e(x) = down_e . (silu(gate_e . x) * (up_e . x)).
 * The whole batch of routed experts in two launches (gate/up, then down)
 * with h kept in device scratch (the guide's API-contract section,
 * coli_vk_expert_group); the
 * routed outputs join each token in rank order and the shared expert last
 * ("colibri -- Vulkan backend (docs/vulkan.md)", the tier's properties and
 * the GLM-5.2 paragraph).  An expert used by several tokens is read once.
 *   ids: int32 [S][k] device; w: f32 [S][k] device; shared: an expert index
 *   or -1 for none; x: f32 [S][H]; y: f32 [S][H]; scratch: device buffer of
 *   at least dqg_expert_group_scratch_bytes(table, S, k) bytes.  After the
 *   call, from byte DQG_SCRATCH_H_OFFSET it
 *   holds h, f32 [S*k + S][I]: slot t*k + r for (token t, rank r), slot
 *   S*k + t for token t's shared expert.
 * An id outside [0, n_experts) makes its token's row of y NaN and sets the
 * scratch flag that dqg_expert_group_take reports.  No host sync.
 */
int dqg_expert_group(const dqg_expert_table *table, int32_t S, int32_t k, const int32_t *ids,
                     const float *w, int32_t shared, const float *x, float *y, void *scratch,
                     size_t scratch_bytes, void *stream);

/*
 * dqg_expert_group with no scratch argument and no allocation, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  The call uses a scratch
 * that the library holds in a static device array of
 * DQG_NOALLOC_SCRATCH_BYTES on each GPU it runs on (until the process ends);
 * the first call on a device takes the array's address there.  It makes no
 * hipMalloc, hipFree or other allocating call; the caller still passes ids,
 * w, x and y.  Calls whose dqg_expert_group_scratch_bytes(table, S, k)
 * exceeds DQG_NOALLOC_SCRATCH_BYTES give DQG_ENOMEM (at I = 2048: up to
 * 2047 slots, S*k + S).  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (other streams, other threads) race, and h
 * and the bad-id flag are not returned.  Runs on the current device, which
 * must be the table's and the stream's.  Otherwise as dqg_expert_group.
 */
#define DQG_NOALLOC_SCRATCH_BYTES (16u << 20)
int dqg_expert_group_noalloc(const dqg_expert_table *table, int32_t S, int32_t k, const int32_t *ids,
                             const float *w, int32_t shared, const float *x, float *y, void *stream);

/* As dqg_expert_group, then records an event in `ticket` (the async form,
 * coli_vk_expert_group_issue in the guide's API-contract section).  The
 * scratch must stay untouched until the ticket is taken. */
int dqg_expert_group_issue(const dqg_expert_table *table, int32_t S, int32_t k,
                           const int32_t *ids, const float *w, int32_t shared, const float *x,
                           float *y, void *scratch, size_t scratch_bytes, void *stream,
                           dqg_ticket *ticket);

/* Join an issued call: waits for its event, then reads its flag.  Returns
 * DQG_OK, DQG_EROUTE (an id was out of range) or DQG_EDEVICE.  Releases
 * the event; a ticket is taken once. */
int dqg_expert_group_take(dqg_ticket *ticket);

/* Router scores (dqg_route's mode). */
typedef enum { DQG_ROUTE_SOFTMAX = 0, DQG_ROUTE_SIGMOID = 1 } dqg_route_mode;

/*
 * The router that feeds dqg_expert_group, on the device: for each token t,
 * scores p from its logits, the k experts of largest pick key, and their
 * weights.  ("colibri -- Vulkan backend (docs/vulkan.md)": the engine
 * tables, whose host rows run the router's softmax and top-k, and MiMo's
 * row: sigmoid scores, a correction bias that picks, the picked weights
 * renormalised; "opus colibri scout": the router row, softmax and top-k in
 * one dispatch.)
 *   mode DQG_ROUTE_SOFTMAX: p[e] = exp(l[e] - max) / sum_j exp(l[j] - max);
 *   mode DQG_ROUTE_SIGMOID: p[e] = 1 / (1 + exp(-l[e]));
 *   pick key: l[e] when bias is NULL (both scores keep the logits' order),
 *   else p[e] + bias[e]; the bias never enters a weight;
 *   ids[t][r], r < k: the picked experts, largest key first, equal keys by
 *   the lower index;
 *   w[t][r] = p[ids[t][r]], divided by the sum of the k picks when renorm,
 *   then times w_scale.
 *   logits: f32 [S][E] device; bias: f32 [E] device or NULL; ids: int32
 *   [S][k] device; w: f32 [S][k] device, the layout dqg_expert_group reads.
 *   1 <= E <= 1024, 1 <= k <= min(E, 64), renorm 0 or 1, w_scale finite.
 *   Logits are expected finite; a NaN logit gives unspecified picks.
 * Checks its arguments before any launch (DQG_EINVAL).  One launch, no
 * host sync; ids and w are ordered with later work on the stream.
 */
int dqg_route(const float *logits, int32_t S, int32_t E, int32_t k, int32_t mode, int32_t renorm,
              const float *bias, float w_scale, int32_t *ids, float *w, void *stream);

/* Per-kernel device time, measured with HIP events that the library
 * records on the launch stream around each kernel it enqueues.
 * dqg_prof_begin(capacity) creates `capacity` event pairs (host-blocking,
 * call it outside timed regions); the next `capacity` launches are timed.
 * dqg_prof_end waits for the recorded events, fills up to `max` records
 * (one per kernel name, in first-launch order), stores their count in *n
 * and releases the events.  Kernel names: "matmul", "gate_up", "gemm",
 * "gemm_gate_up", "gemm_reduce", "dequant", "route", "group_gate_up",
 * "group_act_v4", "group_down". */
typedef struct {
    char kernel[32];
    int64_t launches;
    double total_ms;
} dqg_prof_record;

int dqg_prof_begin(int32_t capacity);
/* dqg_prof_begin that times only the launches of every `every`-th API call
 * (calls counted from this begin, the first one timed), so that a loop pays
 * for the events of 1 call in `every`.  every >= 1; 1 is dqg_prof_begin.
 * On MI355X the launches of a back-to-back loop overlap, and a launch
 * timed among untimed ones reads longer than one timed in a loop where
 * every launch carries events (the events separate the launches). */
int dqg_prof_begin_sampled(int32_t capacity, int32_t every);
int dqg_prof_end(dqg_prof_record *out, int32_t max, int32_t *n);

/* dqg_prof_end launch by launch: fills up to `max` entries in launch order
 * with each timed launch's kernel name and duration, stores their count in
 * *n and releases the events (for percentiles). */
typedef struct {
    char kernel[32];
    double ms;
} dqg_prof_launch;
int dqg_prof_end_launches(dqg_prof_launch *out, int32_t max, int32_t *n);

/*
 * A plain streaming read of nbytes (a positive multiple of 1024) at the
 * 16-byte aligned device pointer p, asynchronous on `stream`: the ceiling
 * that the weight streams are measured against (the bench's streaming-read
 * mode).  Nothing is computed from the bytes but their XOR, which is stored
 * to the 4-byte aligned device word *sink only in the unlikely case that it
 * equals one fixed value.  DQG_EINVAL on a bad argument, DQG_EDEVICE
 * without a device, DQG_ELAUNCH if the launch fails.
 */
int dqg_read_bytes(const void *p, uint64_t nbytes, uint32_t *sink, void *stream);

/* Text of the calling thread's last error (never NULL). *//* Text of the calling thread's last error (never NULL). */
const char *dqg_last_error(void);

/* Snapshot and reset of the process-wide counters. */
void dqg_stats(dqg_counters *out);
void dqg_stats_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* DQG_H */
