// Internal declarations shared by the C-ABI layer (dqg_api.cpp) and the
// kernels (dqg_kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dqg {

// Row pointers of one matrix row: codes, high plane (int3 only), scales.
struct RowPtrs {
    const uint8_t *q;
    const uint8_t *q2;
    const float *s;
};

// A matrix as the kernels see it.
struct MatDev {
    const uint8_t *q;
    const uint8_t *q2;
    const float *s;
    int32_t O, K;
    int32_t qstride;    // bytes of codes per row
    int32_t q2stride;   // bytes of the high plane per row (fmt 5)
    int32_t sstride;    // scales per row of scales
    int32_t shift;      // chunk index >> shift = scale index (31 for one scale a row)
    int32_t srow;       // row >> srow = row of scales (7 for 128-row blocks, else 0)
};

// One expert's matrices in the device table.
struct ExpertDev {
    MatDev gate, up, down;
};

// Codec family a format decodes with (fmt 2 and 4 share the int4 codec,
// fmt 1 and 13 the int8 one).
enum Codec : int { C_I8 = 1, C_I4 = 4, C_I3 = 5, C_FP4 = 7, C_F32 = 10, C_BF16 = 11, C_FP8 = 12, C_F16 = 14 };

// Launch parameters of the grouped expert call.
// The experts' activation: the (clamped) SwiGLU, or DeepSeek V4's rounding
// form of it (I a multiple of 128).
constexpr int32_t ACT_SWIGLU = 0, ACT_SWIGLU_V4 = 1;

struct GroupArgs {
    const ExpertDev *table;
    int32_t n_experts;
    int32_t S, k;
    const int32_t *ids;
    const float *w;
    int32_t shared;      // expert index or -1
    const float *x;      // [S][H]
    float *y;            // [S][H]
    float *h;            // [S*k + S][I]
    int32_t *flag;       // cleared by the gate_up launch, set by the down launch
                         // when an id is out of range
    int32_t H, I;
    float limit;         // swiglu_limit of the experts' SwiGLU, +inf for none
    int32_t act;         // ACT_SWIGLU or ACT_SWIGLU_V4
};

// Launch parameters of the router.
constexpr int ROUTE_MAX_E = 1024;   // experts per token the router kernel holds
struct RouteArgs {
    const float *logits;   // [S][E]
    int32_t S, E, k;
    int32_t mode;          // 0 softmax, 1 sigmoid
    int32_t renorm;        // 1: picked weights divided by their sum
    const float *bias;     // [E] pick bias or null
    float w_scale;
    int32_t *ids;          // [S][k]
    float *w;              // [S][k]
};

// Optional event timing of launches (dqg_api.cpp): when timing is on,
// prof_slot hands out the start/stop events the next launch of `kernel`
// records (hipExtLaunchKernelGGL attaches them to the dispatch itself);
// otherwise it returns false and the launch carries no events.
bool prof_slot(const char *kernel, hipEvent_t *start, hipEvent_t *stop);

// Bytes of the per-device scratch that dqg_expert_group_noalloc uses (a
// static device array in dqg_kernels.hip; DQG_NOALLOC_SCRATCH_BYTES in dqg.h).
constexpr size_t STATIC_SCRATCH_BYTES = size_t(16) << 20;

// The current device's copy of that array (its address taken once per
// device with hipGetSymbolAddress, on the first call made there).
hipError_t static_scratch(void **ptr);

// Host launchers (dqg_kernels.hip).  Return hipSuccess or the launch error.
hipError_t launch_matmul(int codec, const MatDev &m, const float *x, int S, float *y,
                         hipStream_t st);
hipError_t launch_gate_up(int codec, const MatDev &g, const MatDev &u, const float *x, int S,
                          float *h, float limit, hipStream_t st);   // limit: swiglu_limit, +inf for none
hipError_t launch_dequant(int codec, const MatDev &m, float *out, hipStream_t st);
hipError_t launch_read(const void *p, uint64_t nbytes, uint32_t *sink, int cus, hipStream_t st);
hipError_t launch_route(const RouteArgs &a, hipStream_t st);
hipError_t launch_group(int codec_gu, int codec_down, const GroupArgs &a, hipStream_t st,
                        int *launches);

}  // namespace dqg
