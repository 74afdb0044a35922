// Quantised GEMV, SwiGLU gate_up and routed-expert kernels for gfx950 (CDNA4).
//
// What is computed (pages: "colibri Vulkan compute backend complete guide",
// shader-level and API-contract sections; "colibri -- Vulkan backend
// (docs/vulkan.md)", arithmetic paragraph and expert-tier properties):
// weights are decoded from their packed codes and multiplied by f32
// activations; gate_up is silu(gate(x)) * up(x); the expert group sums each
// token's routed experts in rank order, weighted by the router, then adds
// the shared expert.
//
// How, on CDNA4 (prior-art shaders used one subgroup per row, x staged in
// shared memory and one subgroupAdd per row; this keeps the parts that
// hold on a wave64 part with 16-byte loads and DPP):
//  * One wave owns R rows (R rows of gate plus R of up for gate_up).  Lane
//    l streams 16-byte chunks l, l+64, l+128, ... of each row, so a wave's
//    loads of one chunk index are one fully coalesced 1 KiB read per row.
//    All R rows' chunks are issued before any is decoded.
//  * A chunk is decoded in registers into unsigned codes (v_perm and
//    v_cvt_f32_ubyte) and dotted with the matching slice of x for every
//    token of the batch; each decoded weight serves all tokens.  The offset
//    (8 for int4, 4 for int3, 128 for int8 read as offset binary) is folded
//    out once per chunk as OFF * sum(x slice), and the group scale is
//    applied once per chunk, not once per weight.
//  * Per-lane partial sums are reduced across the wave with DPP (quad
//    permutes, row rotates, row broadcasts): no LDS, no barrier.
//  * Every output's arithmetic is the same whatever the batch size, so a
//    token's results have the same bits alone or in a batch.
#include "dqg_internal.h"

#include <hip/hip_ext.h>

#include <mutex>
#include <type_traits>

namespace dqg {
namespace {

constexpr int WAVE = 64;

// Tile shapes of the grouped launches (the measured best on MI355X for the
// int4-g32 group at 1-4 tokens).  Kernel B's 12 rows: 6144 rows make 512
// blocks, one round at two 8-wave blocks per CU (8 rows took 1.5 rounds, 6
// rows two).
constexpr int RA = 4;      // rows of gate (and of up) per wave in kernel A
constexpr int WPB_A = 4;   // waves per block in kernel A
constexpr int RB = 12;     // rows of down per block in kernel B
// Kernel B's blocks in one round (two a CU on 256 CUs), and its row count for
// hidden sizes past 512 blocks of RB: 14 rows keep 6145-7168 rows in one
// round (measured on MI355X, MXFP4 top-8 of 384, H 7168, 8 tokens,
// interleaved: down 144.6-146.2 us in 512 blocks of 14 rows against
// 158.5-162.6 in 598 of 12, although the 14-row kernel spills at the 4-wave
// budget; 16 rows, 448 blocks: 210-211 us).
constexpr int DOWN_ROUND = 512;
constexpr int RB_WIDE = 14;

// Global-memory loads: base pointers are wave-uniform, offsets 32-bit, so
// the address is one SGPR pair plus one VGPR (no per-row 64-bit math).
#define GLOBAL __attribute__((address_space(1)))
typedef const GLOBAL uint8_t *gbytes;
typedef const GLOBAL float *gfloats;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Weight codes are read once per call, so their loads are non-temporal:
// they do not displace x, h and the descriptors in the caches (measured on
// MI355X: the int4-g32 group's gate/up launch 29.3 -> 28.2 us at 1 token;
// a plain read of the same bytes 24.0 -> 22.3 us).
__device__ __forceinline__ uint4 ld16(gbytes base, uint32_t off) {
    const GLOBAL u32x4 *p = (const GLOBAL u32x4 *)(base + off);
    const u32x4 v = __builtin_nontemporal_load(p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld8(gbytes base, uint32_t off) {
    const u32x2 v = *(const GLOBAL u32x2 *)(base + off);
    return make_uint2(v.x, v.y);
}
// idx counts floats; the byte offset is formed in 32 bits
__device__ __forceinline__ float4 ldf4(gfloats base, uint32_t idx) {
    const f32x4 v = *(const GLOBAL f32x4 *)((gbytes)base + (idx << 2));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float ldf(gfloats base, uint32_t idx) {
    return *(const GLOBAL float *)((gbytes)base + (idx << 2));
}
// A weight scale: read once per call, like the codes (measured on MI355X:
// the int4-g32 group's gate/up launch 28.5 -> 28.0 us at 1 token).
__device__ __forceinline__ float ld_scale(gfloats base, uint32_t idx) {
    return __builtin_nontemporal_load((const GLOBAL float *)((gbytes)base + (idx << 2)));
}

// Where a step reads x from: global memory (L2) or the block's LDS copy.
#define LDS __attribute__((address_space(3)))
typedef LDS float *lfloats_w;
typedef const LDS float *lfloats;

// Layout of x in LDS.  A wave's lanes read x one code chunk apart (CW
// inputs: 128 bytes for int4 and MXFP4, 256 for int3), which at those
// strides puts every lane of a 16-byte read on the same LDS banks.  In LDS
// each chunk's slice of x is therefore followed by 4 floats of padding:
// lane strides of 144 and 272 bytes reach every bank (measured on MI355X:
// 127 -> 35 cycles per wave-wide 16-byte read at a 128-byte stride, 257 at
// 256 bytes).  Chunks of 16 inputs (a 64-byte stride, 2-way conflicts)
// stay unpadded: the padding's address arithmetic cost the one-token int8
// launch its register budget.  Chunks of 8 or fewer are conflict-free.
// The expert group's gate/up launch stages x unpadded (P false): there the
// 12% more LDS per block costs a resident block per CU with 2 tokens (3 x
// 48 KB fit 160 KB, 3 x 54 KB do not; measured 54 against 62 us at 2
// tokens), and at 1 token it measured the same either way.
template <int CW, bool P = true>
__host__ __device__ constexpr int x_pad() { return P && CW >= 32 ? 4 : 0; }
// LDS floats of n inputs of x (n a multiple of CW), and the LDS index of input k
template <int CW, bool P = true>
__host__ __device__ constexpr int x_lds_len(int n) { return n + x_pad<CW, P>() * (n / CW); }
template <int CW, bool P = true>
__device__ __forceinline__ uint32_t x_lds_at(uint32_t k) { return k + x_pad<CW, P>() * (k / CW); }
constexpr bool GROUP_XPAD = false;

struct XGlobal {
    gfloats p;
    // 4 inputs at offset off (a multiple of 4) of chunk cu
    template <int CW>
    __device__ __forceinline__ float4 load4(uint32_t cu, uint32_t off) const { return ldf4(p, cu * CW + off); }
};

// A wave-uniform global pointer, held in SGPRs.
__device__ __forceinline__ uint64_t uniform_bits(const void *p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ gbytes gb(const void *p) { return (gbytes)uniform_bits(p); }
__device__ __forceinline__ gfloats gf(const void *p) { return (gfloats)uniform_bits(p); }

// Row pointers as the kernels use them (global address space, uniform).
struct GRow {
    gbytes q, q2;
    gfloats s;
};

// Hides a value's known bits from the optimiser (no instruction).
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
    asm("" : "+v"(x));
    return x;
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// acc + f16(pair half) * x: the f16 -> f32 widening folds into v_fma_mix_f32.
__device__ __forceinline__ float fma_lo(uint32_t pair, float x, float acc) {
    return fmaf((float)__builtin_bit_cast(half2_t, pair).x, x, acc);
}
__device__ __forceinline__ float fma_hi(uint32_t pair, float x, float acc) {
    return fmaf((float)__builtin_bit_cast(half2_t, pair).y, x, acc);
}

// ---------------------------------------------------------------------------
// Codecs.  A chunk is the 16 bytes of codes (plus 8 of high plane for int3)
// one lane reads per step, covering CW inputs.  Unit u of a chunk is inputs
// u * UW .. u * UW + UW - 1; the products of a unit are summed in the order
// IDX gives (a codec's natural decode order), in every kernel alike.
//
// WIDE codecs decode to f32 values, decode_f(ch, u, v): v[i] multiplies
// x[unit base + IDX[i]], with plain f32 FMAs:
//  - int8 (read as offset binary n = q + 128) and int3 give the code
//    itself as a float, byte by byte with v_cvt_f32_ubyte0..3 after the
//    codes are spread one a byte;
//  - MXFP4 converts pairs of e2m1 codes with v_cvt_scalef32_pk_f32_fp4 at
//    scale 1, E4M3 pairs with v_cvt_pk_f32_fp8, bf16 and f32 by bit moves.
// All of these are exact, so weight = (value - OFFS) * VMUL * scale.
// On MI355X v_fmac_f32 issues at about 1.5 times the rate of v_fma_mix_f32
// (an f16 operand converted inside the FMA), so converting each code once
// and using plain FMAs pays the more tokens share a conversion.
//
// The non-WIDE codecs hand decode(ch, u, pr) UW/2 pairs of f16s; half h of
// pair p multiplies x[unit base + IDX[2p + h]] through v_fma_mix_f32 (exact
// f16 -> f32 inside the FMA): f16 rows as they stand, and int4 codes as the
// f16 subnormals n * 2^-24 at one token (a mixed FMA and a cheap pair
// decode beat a conversion and an FMA a product there, measured on the
// one-token expert group); int4 also has decode_f, the same values as f32,
// for several tokens.
//
// SCALED is false for the formats without scales (f32, bf16, f16 rows):
// their scale is the constant 1 and no scale is read.  f32 denormals are
// kept (IEEE mode).
// ---------------------------------------------------------------------------
template <int C>
struct Codec;

// The float value of byte B of w (v_cvt_f32_ubyteB).  w must come from
// opaque() so that the compiler does not fold a mask that made w into a
// bit-field extract ahead of the conversion.
template <int B>
__device__ __forceinline__ float ubyte_f(uint32_t w) {
    return (float)((w >> (8 * B)) & 0xFFu);
}

// int8 rows: byte = two's complement q; q ^ 0x80 = q + 128 as an unsigned
// byte (offset binary), converted byte by byte.
template <>
struct Codec<C_I8> {
    static constexpr int CW = 16, UNITS = 4, UW = 4;
    static constexpr bool F32DEC = false, WIDE = true, SCALED = true;
    static constexpr float VMUL = 1.f, OFFS = 128.f;
    static constexpr int IDX[UW] = {0, 2, 1, 3};
    struct Chunk { uint32_t w[4]; };
    __device__ static Chunk load(const GRow &r, uint32_t c) {
        uint4 v = ld16(r.q, c * 16u);
        return {{v.x, v.y, v.z, v.w}};
    }
    __device__ static void decode_f(const Chunk &ch, int u, float (&v)[UW]) {
        const uint32_t w = opaque(ch.w[u] ^ 0x80808080u);
        v[0] = ubyte_f<0>(w); v[1] = ubyte_f<2>(w); v[2] = ubyte_f<1>(w); v[3] = ubyte_f<3>(w);
    }
};

// int4: nibble i of word u is input 8u + i, decoded two ways with the same
// values:
//  - decode: pairs j = nibbles j, j+4 (they sit at the same offset of the
//    two 16-bit halves) as f16 subnormals n * 2^-24, for v_fma_mix_f32;
//  - decode_f: the same n * 2^-24 as f32 (one mask keeps the even nibbles,
//    one a byte, a shift and the same mask the odd ones; v_cvt_f32_ubyte;
//    an exact scaling), for several tokens, which share each conversion.
template <>
struct Codec<C_I4> {
    static constexpr int CW = 32, UNITS = 4, UW = 8;
    static constexpr bool WIDE = false, F32DEC = true, SCALED = true;
    static constexpr float VMUL = 16777216.f, OFFS = 8.f / 16777216.f;
    static constexpr int IDX[UW] = {0, 4, 1, 5, 2, 6, 3, 7};
    struct Chunk { uint32_t w[4]; };
    __device__ static Chunk load(const GRow &r, uint32_t c) {
        uint4 v = ld16(r.q, c * 16u);
        return {{v.x, v.y, v.z, v.w}};
    }
    __device__ static void decode(const Chunk &ch, int u, uint32_t (&pr)[UW / 2]) {
        const uint32_t w = ch.w[u];
        pr[0] = w & 0x000F000Fu;
        pr[1] = (w >> 4) & 0x000F000Fu;
        pr[2] = (w >> 8) & 0x000F000Fu;
        // each 16-bit half shifted by 12 keeps only its top nibble: one
        // packed 16-bit shift and no mask
        pr[3] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, w) >> (unsigned short)12);
    }
    __device__ static void decode_f(const Chunk &ch, int u, float (&v)[UW]) {
        const uint32_t w = ch.w[u];
        const uint32_t ev = opaque(w & 0x0F0F0F0Fu);          // nibbles 0, 2, 4, 6
        const uint32_t od = opaque((w >> 4) & 0x0F0F0F0Fu);   // nibbles 1, 3, 5, 7
        v[0] = ubyte_f<0>(ev); v[1] = ubyte_f<2>(ev); v[2] = ubyte_f<0>(od); v[3] = ubyte_f<2>(od);
        v[4] = ubyte_f<1>(ev); v[5] = ubyte_f<3>(ev); v[6] = ubyte_f<1>(od); v[7] = ubyte_f<3>(od);
#pragma unroll
        for (int i = 0; i < UW; ++i) v[i] *= 0x1p-24f;
    }
};

// MXFP4: e2m1 codes in int4 order (nibble i of word u is input 8u + i, the
// sign in bit 3), two codes (one byte) per conversion.
typedef float f32x2 __attribute__((ext_vector_type(2)));
template <>
struct Codec<C_FP4> {
    static constexpr int CW = 32, UNITS = 4, UW = 8;
    static constexpr bool F32DEC = false, WIDE = true, SCALED = true;
    static constexpr float VMUL = 1.f, OFFS = 0.f;
    static constexpr int IDX[UW] = {0, 1, 2, 3, 4, 5, 6, 7};
    struct Chunk { uint32_t w[4]; };
    __device__ static Chunk load(const GRow &r, uint32_t c) {
        uint4 v = ld16(r.q, c * 16u);
        return {{v.x, v.y, v.z, v.w}};
    }
    __device__ static void decode_f(const Chunk &ch, int u, float (&v)[UW]) {
        const uint32_t w = ch.w[u];
        const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);   // byte 0: inputs 0, 1
        const f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
        const f32x2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
        const f32x2 d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
        v[0] = a.x; v[1] = a.y; v[2] = b.x; v[3] = b.y; v[4] = c.x; v[5] = c.y; v[6] = d.x; v[7] = d.y;
    }
};

// int3-g64: a chunk is one group of 64 inputs: 16 bytes of the 2-bit plane
// (words L0..L3, 16 inputs each) and 8 bytes of the 1-bit plane (H0, H1, 32
// inputs each).  Unit u is inputs 32u..32u+31: L(2u), L(2u+1), H(u).  For
// m = 0..7, byte b of q_m is the 3-bit code of input 8b + m: the 2-bit
// fields are gathered with one v_perm per four m, the high bits with a
// shift, the two joined with a shift-or, and each byte of q_m converted.
template <>
struct Codec<C_I3> {
    static constexpr int CW = 64, UNITS = 2, UW = 32;
    static constexpr bool F32DEC = false, WIDE = true, SCALED = true;
    static constexpr float VMUL = 1.f, OFFS = 4.f;
    // v[4m + b] is input 8b + m
    static constexpr int IDX[UW] = {0, 8, 16, 24, 1, 9, 17, 25, 2, 10, 18, 26, 3, 11, 19, 27,
                                    4, 12, 20, 28, 5, 13, 21, 29, 6, 14, 22, 30, 7, 15, 23, 31};
    struct Chunk { uint32_t l[4]; uint32_t h[2]; };
    __device__ static Chunk load(const GRow &r, uint32_t c) {
        uint4 lv = ld16(r.q, c * 16u);
        uint2 hv = ld8(r.q2, c * 8u);
        return {{lv.x, lv.y, lv.z, lv.w}, {hv.x, hv.y}};
    }
    __device__ static void decode_f(const Chunk &ch, int u, float (&v)[UW]) {
        const uint32_t L0 = ch.l[2 * u], L1 = ch.l[2 * u + 1], H = ch.h[u];
        // za = [L0.b0, L0.b2, L1.b0, L1.b2]: fields of inputs m, 8+m, 16+m, 24+m (m < 4)
        // zb = [L0.b1, L0.b3, L1.b1, L1.b3]: the same for m >= 4
        const uint32_t za = __builtin_amdgcn_perm(L1, L0, 0x06040200u);
        const uint32_t zb = __builtin_amdgcn_perm(L1, L0, 0x07050301u);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const uint32_t z = m < 4 ? za : zb;
            const uint32_t lo = (z >> (2 * (m & 3))) & 0x03030303u;
            const uint32_t hi = (H >> m) & 0x01010101u;
            const uint32_t q = opaque(lo | (hi << 2));
            v[4 * m] = ubyte_f<0>(q); v[4 * m + 1] = ubyte_f<1>(q);
            v[4 * m + 2] = ubyte_f<2>(q); v[4 * m + 3] = ubyte_f<3>(q);
        }
    }
};

// f16 rows: the words are already f16 pairs, the even input in the low half.
template <>
struct Codec<C_F16> {
    static constexpr int CW = 8, UNITS = 2, UW = 4;
    static constexpr bool F32DEC = false, WIDE = false, SCALED = false;
    static constexpr float VMUL = 1.f, OFFS = 0.f;
    static constexpr int IDX[UW] = {0, 1, 2, 3};
    struct Chunk { uint32_t w[4]; };
    __device__ static Chunk load(const GRow &r, uint32_t c) {
        uint4 v = ld16(r.q, c * 16u);
        return {{v.x, v.y, v.z, v.w}};
    }
    __device__ static void decode(const Chunk &ch, int u, uint32_t (&pr)[UW / 2]) {
        pr[0] = ch.w[2 * u];
        pr[1] = ch.w[2 * u + 1];
    }
};

// f32 rows: four values a chunk, read as they are.
template <>
struct Codec<C_F32> {
    static constexpr int CW = 4, UNITS = 1, UW = 4;
    static constexpr bool F32DEC = false, WIDE = true, SCALED = false;
    static constexpr float VMUL = 1.f, OFFS = 0.f;
    static constexpr int IDX[UW] = {0, 1, 2, 3};
    struct Chunk { uint32_t w[4]; };
    __device__ static Chunk load(const GRow &r, uint32_t c) {
        uint4 v = ld16(r.q, c * 16u);
        return {{v.x, v.y, v.z, v.w}};
    }
    __device__ static void decode_f(const Chunk &ch, int, float (&v)[UW]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(ch.w[i]);
    }
};

// bf16 rows: a bf16 is the upper half of an f32, so each half of a word
// becomes an f32 by one shift or one mask (even input in the low half).
template <>
struct Codec<C_BF16> {
    static constexpr int CW = 8, UNITS = 2, UW = 4;
    static constexpr bool F32DEC = false, WIDE = true, SCALED = false;
    static constexpr float VMUL = 1.f, OFFS = 0.f;
    static constexpr int IDX[UW] = {0, 1, 2, 3};
    struct Chunk { uint32_t w[4]; };
    __device__ static Chunk load(const GRow &r, uint32_t c) {
        uint4 v = ld16(r.q, c * 16u);
        return {{v.x, v.y, v.z, v.w}};
    }
    __device__ static void decode_f(const Chunk &ch, int u, float (&v)[UW]) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t w = ch.w[2 * u + j];
            v[2 * j] = __uint_as_float(w << 16);
            v[2 * j + 1] = __uint_as_float(w & 0xFFFF0000u);
        }
    }
};

// E4M3 (OCP FP8) with one f32 scale per 128 x 128 block: v_cvt_pk_f32_fp8
// turns two codes into two f32 values, exactly (NaN codes stay NaN).
template <>
struct Codec<C_FP8> {
    static constexpr int CW = 16, UNITS = 4, UW = 4;
    static constexpr bool F32DEC = false, WIDE = true, SCALED = true;
    static constexpr float VMUL = 1.f, OFFS = 0.f;
    static constexpr int IDX[UW] = {0, 1, 2, 3};
    struct Chunk { uint32_t w[4]; };
    __device__ static Chunk load(const GRow &r, uint32_t c) {
        uint4 v = ld16(r.q, c * 16u);
        return {{v.x, v.y, v.z, v.w}};
    }
    __device__ static void decode_f(const Chunk &ch, int u, float (&v)[UW]) {
        const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(ch.w[u], false);   // bytes 0, 1
        const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(ch.w[u], true);    // bytes 2, 3
        v[0] = a.x; v[1] = a.y; v[2] = b.x; v[3] = b.y;
    }
};

// Whether a step over SM tokens multiplies f32 values (decode_f) rather than
// f16 pairs: the WIDE codecs always, int4 from two tokens up (one
// conversion then serves every token; at one token v_fma_mix_f32's
// conversion inside the FMA is the cheaper form).  Both forms hold the same
// values, so the bits do not depend on the form.
template <int C, int SM>
constexpr bool dec_f32() { return Codec<C>::WIDE || (Codec<C>::F32DEC && SM >= 2); }

// ---------------------------------------------------------------------------
// Wave64 sum with DPP.  Quad permutes and row rotates give every lane its
// row's sum; two row broadcasts carry rows 0..2 into row 3.  The total is
// read from lane 63 (uniform result).  The order of the additions is fixed.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_rows(float v) {
    // rows outside ROW_MASK read 0
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}

__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_mov<0xB1>(v);        // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E>(v);        // quad_perm [2,3,0,1]
    v += dpp_mov<0x124>(v);       // row_ror:4
    v += dpp_mov<0x128>(v);       // row_ror:8
    v += dpp_rows<0x142, 0xA>(v); // row_bcast:15 into rows 1 and 3
    v += dpp_rows<0x143, 0xC>(v); // row_bcast:31 into rows 2 and 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / WAVE));
}

// silu(z) = z * sigmoid(z), the sigmoid taken from e = exp(-|z|), which lies
// in [0, 1]: no intermediate overflows, so for z < -88.7 (where exp(-z)
// would) the result is still z e^z / (1 + e^z) down to f32's subnormals.
__device__ __forceinline__ float silu(float z) {
    const float e = expf(-fabsf(z));
    const float r = 1.0f / (1.0f + e);
    return z >= 0.f ? z * r : (z * e) * r;
}

// SwiGLU with a limit L (swiglu_limit): silu(min(g, L)) * clamp(u, -L, L).
// L = +inf leaves g and u unchanged, bit for bit; a NaN stays NaN.
__device__ __forceinline__ float swiglu(float g, float u, float L) {
    const float gc = g > L ? L : g;
    const float uc = u > L ? L : (u < -L ? -L : u);
    return silu(gc) * uc;
}

// DeepSeek V4's rounding activation ("colibri -- Vulkan backend
// (docs/vulkan.md)", the paragraph on DeepSeek V4's CPU expert and the
// tier's third activation): bf16 and E4M3 roundings, to nearest, ties to
// even, on the bits.
//
// bf16: add 0x7FFF plus the lowest kept bit, then clear the low 16 bits (a
// carry out of the fraction steps the exponent, as rounding up should).
__device__ __forceinline__ float round_bf16(float v) {
    uint32_t b = __float_as_uint(v);
    if ((b & 0x7F800000u) == 0x7F800000u) return v;   // inf and NaN unchanged
    b += 0x7FFFu + ((b >> 16) & 1u);
    return __uint_as_float(b & 0xFFFF0000u);
}

// E4M3 (1.4.3, bias 7, no infinities) for |v| < 464, where no value rounds
// past 448.  From 2^-6 up: 3 fraction bits, the same carry trick at bit 20;
// below: the subnormal quantum 2^-9 (v * 512 is exact, rintf ties to even).
__device__ __forceinline__ float round_e4m3(float v) {
    const float a = fabsf(v);
    float r;
    if (a < 0x1p-6f) {
        r = rintf(a * 512.f) * 0x1p-9f;
    } else {
        uint32_t b = __float_as_uint(a);
        b += 0x7FFFFu + ((b >> 20) & 1u);
        r = __uint_as_float(b & 0xFFF00000u);
    }
    return copysignf(r, v);
}

// The exponent j of the block scale 2^j: the smallest power of two that
// takes m (the block's largest magnitude) below 448; 0 for m = 0.  With
// m = f 2^e, f in [1/2, 1): m / 2^(e-9) = 512 f lies in [256, 512), so j is
// e - 9 when 512 f < 448 and e - 8 otherwise.
__device__ __forceinline__ int v4_scale_exp(float m) {
    if (!(m > 0.f)) return 0;
    int e;
    const float f = frexpf(m, &e);
    return f * 512.f < 448.f ? e - 9 : e - 8;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// ---------------------------------------------------------------------------
// The row-set dot product.  acc[r][s] (per lane) = this lane's share of
// sum_k W_r[k] * x_s[k]; reduce with wave_sum.  Per chunk and row:
// p = sum(pattern * x) over the chunk, then acc += scale * VMUL *
// (p - OFFS * sum(x)): the code offset is removed once per chunk and the
// scale applied once per chunk.
//
// A step issues every load of one chunk (codes and scales of all rows,
// then x) before any arithmetic, held ahead by a scheduling barrier, so a
// wave has all its requests in flight before it waits.  The chunk index
// is hidden from loop strength reduction so that each load is one SGPR
// base plus a 32-bit lane offset.
// ---------------------------------------------------------------------------
template <int C, int NR, int SM>
struct Step {
    typename Codec<C>::Chunk ch[NR];
    float sc[NR];
    float xv[SM][Codec<C>::CW];
};

// Codes and scales of chunk cu of every row.
template <int C, int NR, int SM>
__device__ __forceinline__ void step_load_w(Step<C, NR, SM> &st, const GRow (&rows)[NR], int shift, uint32_t cu) {
    using Cd = Codec<C>;
    const uint32_t si = cu >> shift;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        st.ch[r] = Cd::load(rows[r], cu);
        st.sc[r] = Cd::SCALED ? ld_scale(rows[r].s, si) : 1.f;
    }
}

// The matching slice of x for every token of the batch.
template <int C, int NR, int SM, typename XP>
__device__ __forceinline__ void step_load_x(Step<C, NR, SM> &st, const XP (&xp)[SM], uint32_t cu) {
    using Cd = Codec<C>;
#pragma unroll
    for (int s = 0; s < SM; ++s)
#pragma unroll
        for (int i = 0; i < Cd::CW / 4; ++i) {
            const float4 t = xp[s].template load4<Cd::CW>(cu, 4 * i);
            st.xv[s][4 * i] = t.x; st.xv[s][4 * i + 1] = t.y; st.xv[s][4 * i + 2] = t.z; st.xv[s][4 * i + 3] = t.w;
        }
}

template <int C, int NR, int SM, typename XP>
__device__ __forceinline__ void step_load(Step<C, NR, SM> &st, const GRow (&rows)[NR], int shift,
                                          const XP (&xp)[SM], uint32_t cu) {
    step_load_w(st, rows, shift, cu);
    step_load_x(st, xp, cu);
}

template <int C, int NR, int SM>
__device__ __forceinline__ void step_compute(const Step<C, NR, SM> &st, float (&acc)[NR][SM]) {
    using Cd = Codec<C>;
    float p[NR][SM], xs[SM];
#pragma unroll
    for (int s = 0; s < SM; ++s) {
        xs[s] = 0.f;
        if (Cd::OFFS != 0.f) {
#pragma unroll
            for (int i = 0; i < Cd::CW; ++i) xs[s] += st.xv[s][i];
        }
#pragma unroll
        for (int r = 0; r < NR; ++r) p[r][s] = 0.f;
    }
#pragma unroll
    for (int u = 0; u < Cd::UNITS; ++u) {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            if constexpr (dec_f32<C, SM>()) {
                float v[Cd::UW];
                Cd::decode_f(st.ch[r], u, v);
#pragma unroll
                for (int s = 0; s < SM; ++s)
#pragma unroll
                    for (int i = 0; i < Cd::UW; ++i) p[r][s] = fmaf(v[i], st.xv[s][u * Cd::UW + Cd::IDX[i]], p[r][s]);
            } else {
                uint32_t pr[Cd::UW / 2];
                Cd::decode(st.ch[r], u, pr);
#pragma unroll
                for (int s = 0; s < SM; ++s)
#pragma unroll
                    for (int q = 0; q < Cd::UW / 2; ++q) {
                        p[r][s] = fma_lo(pr[q], st.xv[s][u * Cd::UW + Cd::IDX[2 * q]], p[r][s]);
                        p[r][s] = fma_hi(pr[q], st.xv[s][u * Cd::UW + Cd::IDX[2 * q + 1]], p[r][s]);
                    }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int s = 0; s < SM; ++s)
            acc[r][s] = fmaf(st.sc[r] * Cd::VMUL, fmaf(-Cd::OFFS, xs[s], p[r][s]), acc[r][s]);
}

// One row of step_compute for one token: the same operations in the same
// order for that row (xs is step_compute's sum of x over the chunk, 0 for
// offset-free codes), so that a caller can compute rows one by one as their
// loads land.
template <int C>
__device__ __forceinline__ float row_dot(const typename Codec<C>::Chunk &ch, float sc,
                                         const float (&xv)[Codec<C>::CW], float xs, float acc) {
    using Cd = Codec<C>;
    float p = 0.f;
#pragma unroll
    for (int u = 0; u < Cd::UNITS; ++u) {
        if constexpr (Cd::WIDE) {
            float v[Cd::UW];
            Cd::decode_f(ch, u, v);
#pragma unroll
            for (int i = 0; i < Cd::UW; ++i) p = fmaf(v[i], xv[u * Cd::UW + Cd::IDX[i]], p);
        } else {
            uint32_t pr[Cd::UW / 2];
            Cd::decode(ch, u, pr);
#pragma unroll
            for (int q = 0; q < Cd::UW / 2; ++q) {
                p = fma_lo(pr[q], xv[u * Cd::UW + Cd::IDX[2 * q]], p);
                p = fma_hi(pr[q], xv[u * Cd::UW + Cd::IDX[2 * q + 1]], p);
            }
        }
    }
    return fmaf(sc * Cd::VMUL, fmaf(-Cd::OFFS, xs, p), acc);
}

template <int C, int NR, int SM, typename XP = XGlobal>
__device__ __forceinline__ void dot_rows(const GRow (&rows)[NR], int nch, int shift,
                                         const XP (&xp)[SM], float (&acc)[NR][SM]) {
    const int lane = threadIdx.x & (WAVE - 1);
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int s = 0; s < SM; ++s) acc[r][s] = 0.f;
    for (int c = lane; c < nch; c += WAVE) {
        Step<C, NR, SM> st;
        step_load(st, rows, shift, xp, opaque((uint32_t)c));
        __builtin_amdgcn_sched_barrier(0);
        step_compute(st, acc);
    }
}

// step_compute with x in LDS: x is read per decode unit (UW values per
// token) as the unit is used, so only SM * UW values of x are live at a
// time instead of SM * CW; the operations and their order are those of
// step_compute, so the results have the same bits.  x + s * xstride is
// token s's row of the staged x.  With XSP the chunk's sums of x come in
// xsp (summed beforehand in the same order) instead of being summed here.
template <int C, int NR, int SM, bool P = true, bool XSP = false>
__device__ __forceinline__ void step_compute_lds(const Step<C, NR, SM> &st, lfloats x, uint32_t xstride,
                                                 uint32_t cu, float (&acc)[NR][SM], const float *xsp = nullptr) {
    using Cd = Codec<C>;
    float p[NR][SM], xs[SM];
#pragma unroll
    for (int s = 0; s < SM; ++s) {
        xs[s] = XSP ? xsp[s] : 0.f;
#pragma unroll
        for (int r = 0; r < NR; ++r) p[r][s] = 0.f;
    }
#pragma unroll
    for (int u = 0; u < Cd::UNITS; ++u) {
        float xv[SM][Cd::UW];
#pragma unroll
        for (int s = 0; s < SM; ++s)
#pragma unroll
            for (int i = 0; i < Cd::UW / 4; ++i) {
                const f32x4 t = *(const LDS f32x4 *)(x + s * xstride + x_lds_at<Cd::CW, P>(cu * Cd::CW) + u * Cd::UW + 4 * i);
                xv[s][4 * i] = t.x; xv[s][4 * i + 1] = t.y; xv[s][4 * i + 2] = t.z; xv[s][4 * i + 3] = t.w;
            }
        if (Cd::OFFS != 0.f && !XSP) {
#pragma unroll
            for (int s = 0; s < SM; ++s)
#pragma unroll
                for (int i = 0; i < Cd::UW; ++i) xs[s] += xv[s][i];
        }
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            if constexpr (dec_f32<C, SM>()) {
                float v[Cd::UW];
                Cd::decode_f(st.ch[r], u, v);
#pragma unroll
                for (int s = 0; s < SM; ++s)
#pragma unroll
                    for (int i = 0; i < Cd::UW; ++i) p[r][s] = fmaf(v[i], xv[s][Cd::IDX[i]], p[r][s]);
            } else {
                uint32_t pr[Cd::UW / 2];
                Cd::decode(st.ch[r], u, pr);
#pragma unroll
                for (int s = 0; s < SM; ++s)
#pragma unroll
                    for (int q = 0; q < Cd::UW / 2; ++q) {
                        p[r][s] = fma_lo(pr[q], xv[s][Cd::IDX[2 * q]], p[r][s]);
                        p[r][s] = fma_hi(pr[q], xv[s][Cd::IDX[2 * q + 1]], p[r][s]);
                    }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int s = 0; s < SM; ++s)
            acc[r][s] = fmaf(st.sc[r] * Cd::VMUL, fmaf(-Cd::OFFS, xs[s], p[r][s]), acc[r][s]);
}

// step_compute_lds for one token, rows in pairs: all units of a pair before
// the next pair, so that a pair's arithmetic waits only for its own rows'
// loads (a step's loads go out in row order) and arithmetic overlaps the
// arrival of the later rows.  x is read again per pair; the chunk's sum of x
// (for the code offset) comes from LDS, summed at staging in the order
// step_compute and step_compute_lds sum it, so the bits are theirs.
template <int C, int NR, bool P>
__device__ __forceinline__ void step_compute_lds_pairs(const Step<C, NR, 1> &st, lfloats x, float xsum, uint32_t cu,
                                                       float (&acc)[NR][1]) {
    using Cd = Codec<C>;
    static_assert(NR % 2 == 0, "rows in pairs");
#pragma unroll
    for (int r0 = 0; r0 < NR; r0 += 2) {
        float p[2] = {0.f, 0.f};
#pragma unroll
        for (int u = 0; u < Cd::UNITS; ++u) {
            float xv[Cd::UW];
#pragma unroll
            for (int i = 0; i < Cd::UW / 4; ++i) {
                const f32x4 t = *(const LDS f32x4 *)(x + x_lds_at<Cd::CW, P>(cu * Cd::CW) + u * Cd::UW + 4 * i);
                xv[4 * i] = t.x; xv[4 * i + 1] = t.y; xv[4 * i + 2] = t.z; xv[4 * i + 3] = t.w;
            }
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                if constexpr (Cd::WIDE) {
                    float v[Cd::UW];
                    Cd::decode_f(st.ch[r0 + rr], u, v);
#pragma unroll
                    for (int i = 0; i < Cd::UW; ++i) p[rr] = fmaf(v[i], xv[Cd::IDX[i]], p[rr]);
                } else {
                    uint32_t pr[Cd::UW / 2];
                    Cd::decode(st.ch[r0 + rr], u, pr);
#pragma unroll
                    for (int q = 0; q < Cd::UW / 2; ++q) {
                        p[rr] = fma_lo(pr[q], xv[Cd::IDX[2 * q]], p[rr]);
                        p[rr] = fma_hi(pr[q], xv[Cd::IDX[2 * q + 1]], p[rr]);
                    }
                }
            }
        }
#pragma unroll
        for (int rr = 0; rr < 2; ++rr)
            acc[r0 + rr][0] = fmaf(st.sc[r0 + rr] * Cd::VMUL, fmaf(-Cd::OFFS, xsum, p[rr]), acc[r0 + rr][0]);
    }
}

// Whether the one-token group path takes its rows in pairs (and so stages
// the chunk sums of x): an even row count.
template <int C, int NR>
constexpr bool gu1_pairs() { return NR % 2 == 0; }

// dot_rows for one token with x in LDS, when the caller has already issued
// the codes and scales of this lane's first chunk into st (have: this lane
// has a first chunk), e.g. before staging x, so that both latencies overlap.
// xsum: the chunk sums of x (used with gu1_pairs).
// A wave computes each step at raised priority, so that a wave whose bytes
// have arrived finishes the step and requests its next one ahead of waves
// still waiting (measured on MI355X: the int4-g32 group's gate/up launch
// 28.1-28.2 -> 27.4-27.5 us at 1 token).
template <int C, int NR>
__device__ __forceinline__ void dot_rows_lds1(Step<C, NR, 1> &st, bool have, const GRow (&rows)[NR], int nch,
                                              int shift, lfloats x, lfloats xsum, float (&acc)[NR][1]) {
    const int lane = threadIdx.x & (WAVE - 1);
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[r][0] = 0.f;
    for (int c = lane; c < nch; c += WAVE) {
        const uint32_t cu = opaque((uint32_t)c);
        if (!(have && c == lane)) step_load_w(st, rows, shift, cu);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
        if constexpr (gu1_pairs<C, NR>())
            step_compute_lds_pairs<C, NR, GROUP_XPAD>(st, x, Codec<C>::OFFS != 0.f ? xsum[cu] : 0.f, cu, acc);
        else
            step_compute_lds<C, NR, 1, GROUP_XPAD>(st, x, 0u, cu, acc);
        __builtin_amdgcn_s_setprio(0);
    }
}

// Pointers of one row.  Rows are wave-uniform in every kernel but dequant;
// readfirstlane keeps them in SGPRs even when the matrix came from a table
// read with vector loads.
__device__ __forceinline__ GRow row_ptrs(const MatDev &m, int row) {
    return {gb(m.q + (size_t)row * m.qstride), gb(m.q2 + (size_t)row * m.q2stride),
            gf(m.s + (size_t)(row >> m.srow) * m.sstride)};
}

// Pointers of a row that may differ from lane to lane (the dequant kernel).
__device__ __forceinline__ GRow lane_row_ptrs(const MatDev &m, int row) {
    return {(gbytes)(m.q + (size_t)row * m.qstride), (gbytes)(m.q2 + (size_t)row * m.q2stride),
            (gfloats)(m.s + (size_t)(row >> m.srow) * m.sstride)};
}

// ---------------------------------------------------------------------------
// dqg_matmul and dqg_gate_up, per-row route (up to 8 tokens a pass)
// ---------------------------------------------------------------------------
// dqg_matmul (GU false: y[s][o] = W[o] . x[s], W = m0) and dqg_gate_up
// (GU true: y[s][i] = swiglu(G[i] . x[s], U[i] . x[s]), G = m0, U = m1)
// with x staged in LDS, K-chunk by K-chunk: the block's waves share one copy
// of x instead of each reading it from L2.  A K-chunk is a multiple of 64
// code chunks, so every lane takes chunks lane, lane + 64, ... in order
// whatever the K-chunk and the batch: a token's bits do not depend on S.
// Every wave stays to the end (block barriers); rows past O are clamped and
// their outputs dropped.
template <int C, int R, int SM, bool GU>
__global__ void __launch_bounds__(256) k_rows_lds(MatDev m0, MatDev m1, const float *__restrict__ x, int S,
                                                  float *__restrict__ y, int KC, float L) {
    extern __shared__ float xl_raw[];
    lfloats_w xs = (lfloats_w)xl_raw;
    using Cd = Codec<C>;
    constexpr int NR = GU ? 2 * R : R;   // GU: gate rows, then the same rows of up
    const MatDev &m = m0;
    const int wave = blockIdx.x * (blockDim.x / WAVE) + wave_id();
    const int row0 = wave * R;
    const int lane = threadIdx.x & (WAVE - 1);
    GRow rows[NR];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        rows[r] = row_ptrs(m0, min(row0 + r, m.O - 1));
        if (GU) rows[R + r] = row_ptrs(m1, min(row0 + r, m.O - 1));
    }
    for (int s0 = 0; s0 < S; s0 += SM) {
        float acc[NR][SM];
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int s = 0; s < SM; ++s) acc[r][s] = 0.f;
        for (int kc0 = 0; kc0 < m.K; kc0 += KC) {
            const int kn = min(KC, m.K - kc0), n4 = kn / 4;
            const int c0 = kc0 / Cd::CW, nc = kn / Cd::CW;
            // this lane's first step of the chunk is requested before x is
            // staged, so that the two round trips overlap
            Step<C, NR, SM> st;
            if (lane < nc) step_load_w(st, rows, m.shift, opaque((uint32_t)lane) + (uint32_t)c0);
            __syncthreads();   // the previous chunk's readers are done
            for (int i0 = threadIdx.x; i0 < SM * n4; i0 += 8 * (int)blockDim.x) {
                f32x4 v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int i = i0 + u * (int)blockDim.x, sl = i / n4, k4 = i - sl * n4;
                    v[u] = (i < SM * n4 && s0 + sl < S)
                               ? *(const GLOBAL f32x4 *)(gf(x) + (size_t)(s0 + sl) * m.K + kc0 + 4 * k4)
                               : f32x4{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int i = i0 + u * (int)blockDim.x, sl = i / n4, k4 = i - sl * n4;
                    if (i < SM * n4) *(LDS f32x4 *)(xs + (size_t)sl * x_lds_len<Cd::CW>(KC) + x_lds_at<Cd::CW>(4 * k4)) = v[u];
                }
            }
            __syncthreads();
            for (int c = lane; c < nc; c += WAVE) {
                const uint32_t cu = opaque((uint32_t)c);
                if (c != lane) step_load_w(st, rows, m.shift, cu + (uint32_t)c0);
                __builtin_amdgcn_sched_barrier(0);
                step_compute_lds(st, (lfloats)xs, (uint32_t)x_lds_len<Cd::CW>(KC), cu, acc);
            }
        }
        float out = 0.f, outu = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int s = 0; s < SM; ++s) {
                const float t = wave_sum(acc[r][s]);
                const float tu = GU ? wave_sum(acc[R + r][s]) : 0.f;
                if (lane == r * SM + s) { out = t; outu = tu; }
            }
        const int r = lane / SM, s = lane % SM;
        if (lane < R * SM && row0 + r < m.O && s0 + s < S)
            y[(size_t)(s0 + s) * m.O + row0 + r] = GU ? swiglu(out, outu, L) : out;
    }
}

// The same products for 1-4 tokens (int3: 1) and K of 1-4 whole 64-chunk steps (NS),
// shaped to fill the chip at one token: blocks of 12 waves x 1 row (6144
// rows make 512 blocks, two a CU; int3, and the single expert's launches,
// 12 waves x 2 rows), x staged once per block, and every
// weight load of a wave issued before its first arithmetic.  x's loads go
// out first; at one token the weights' loads (step by step, rows in order)
// follow once x is in LDS, at several tokens while x is in flight; then
// each row of each step is computed as its codes land (one token: the
// step's x in registers; more, or int3: step_compute_lds).  The per-row
// arithmetic and the order of steps are k_rows_lds's, so the bits are the
// same.
constexpr int GX_W = 12, GX_R = 2;
// One token with codes of at most 32 inputs a chunk: one row a wave, so that
// the arithmetic left when a wave's last bytes land is one row's (measured on
// MI355X, interleaved against 12 x 2: 6144^2 int4 6.75-7.07 -> 6.44-6.47 us,
// its gate_up 11.0-11.2 -> 10.5; int3 6144 x 16384, whose rows are longer,
// loses: 12.9-13.4 -> 14.1-14.8).
constexpr int GX1_R = 1;
// Several tokens: 8 waves x 3 rows, so that the x of each chunk a wave reads
// from LDS serves 3 rows (the reads of x for 2-4 tokens cost LDS bandwidth
// on the scale of the arithmetic).
constexpr int GXM_W = 8, GXM_R = 3;
// Matrices of fewer rows take blocks of 8 waves x 1 row, so that 2048 rows
// still make 256 blocks.
constexpr int GXS_W = 8, GXS_R = 1;
constexpr int GX_WIDE_ROWS = 256 * GX_W * GX_R;   // the wide shapes from this many rows up

// The body of k_rows_x for blocks of W waves x R rows (GU: R rows of m0 and
// the same rows of m1).  epi(s, row, v, vu) takes token s's dot product of
// row (and of m1's row with GU), for rows below m0.O and s below S.
// XFIRST: the weights are requested only once x is staged, so that x comes
// back through an idle memory system and the arithmetic starts while the
// weights stream (the dense one-token launches: 6144^2 int4 7.6 -> 7.0 us,
// its gate_up 13.2 -> 10.8, int3 6144 x 16384 15.6 -> 12.9; no gain at 4
// tokens, and the single expert's short launches lose); otherwise they go
// out with x and wait for it.
template <int C, int SM, bool GU, int NS, int W, int R, bool XFIRST, typename Epi>
__device__ __forceinline__ void rows_x_body(const MatDev &m0, const MatDev &m1, const float *__restrict__ x, int S,
                                            Epi &&epi) {
    extern __shared__ float xl_raw[];
    lfloats_w xs = (lfloats_w)xl_raw;
    using Cd = Codec<C>;
    constexpr int NR = GU ? 2 * R : R;
    constexpr int K = NS * WAVE * Cd::CW;                     // m0.K (checked by the launcher)
    constexpr uint32_t k4n = K / 4, n4 = SM * k4n, nt = WAVE * W, XN = (n4 + nt - 1) / nt;
    constexpr uint32_t xl = (uint32_t)x_lds_len<Cd::CW>(K);
    const MatDev &m = m0;
    const int lane = threadIdx.x & (WAVE - 1);
    const int row0 = (blockIdx.x * W + wave_id()) * R;
    // x of every token (a second token past S repeats the first; its outputs are dropped)
    f32x4 xv4[XN];
#pragma unroll
    for (uint32_t u = 0; u < XN; ++u) {
        const uint32_t i = min((uint32_t)threadIdx.x + u * nt, n4 - 1), sl = i / k4n, k4 = i - sl * k4n;
        xv4[u] = *(const GLOBAL f32x4 *)(gf(x) + (size_t)min((int)sl, S - 1) * K + 4 * k4);
    }
    GRow rows[NR];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        rows[r] = row_ptrs(m0, min(row0 + r, m.O - 1));
        if (GU) rows[R + r] = row_ptrs(m1, min(row0 + r, m.O - 1));
    }
    Step<C, NR, SM> st[NS];
    const auto load_weights = [&]() {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            step_load_w(st[j], rows, m.shift, opaque((uint32_t)(j * WAVE + lane)));
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if constexpr (!XFIRST) load_weights();
#pragma unroll
    for (uint32_t u = 0; u < XN; ++u) {
        const uint32_t i = min((uint32_t)threadIdx.x + u * nt, n4 - 1), sl = i / k4n, k4 = i - sl * k4n;
        *(LDS f32x4 *)(xs + sl * xl + x_lds_at<Cd::CW>(4 * k4)) = xv4[u];
    }
    __syncthreads();
    // one token with a chunk of at most 32 inputs takes the step's x in
    // registers; several tokens, and int3's 64-input chunks, read x per
    // decode unit from LDS.  Codes with an offset take each chunk's sum of x
    // per token, summed once per block in step_compute's order, after the row.
    constexpr bool XREG = SM == 1 && Cd::CW <= 32;
    constexpr bool XSUM = Cd::OFFS != 0.f;
    constexpr uint32_t NCH = K / Cd::CW;
    lfloats_w xsums = xs + SM * xl;
    if constexpr (XSUM) {
        for (uint32_t t = threadIdx.x; t < SM * NCH; t += nt) {
            const uint32_t sl = t / NCH, c = t - sl * NCH;
            float a = 0.f;
#pragma unroll
            for (int q = 0; q < Cd::CW / 4; ++q) {
                const f32x4 v = *(const LDS f32x4 *)(xs + sl * xl + x_lds_at<Cd::CW>(c * Cd::CW) + 4 * q);
                a += v.x;
                a += v.y;
                a += v.z;
                a += v.w;
            }
            xsums[t] = a;
        }
        __syncthreads();
    }
    if constexpr (XFIRST) load_weights();
    float acc[NR][SM];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int s = 0; s < SM; ++s) acc[r][s] = 0.f;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const uint32_t cu = (uint32_t)(j * WAVE + lane);
        if constexpr (XREG) {
            float xv[Cd::CW];
#pragma unroll
            for (int q = 0; q < Cd::CW / 4; ++q) {
                const f32x4 t = *(const LDS f32x4 *)(xs + x_lds_at<Cd::CW>(cu * Cd::CW) + 4 * q);
                xv[4 * q] = t.x; xv[4 * q + 1] = t.y; xv[4 * q + 2] = t.z; xv[4 * q + 3] = t.w;
            }
            const float xsum = XSUM ? xsums[cu] : 0.f;
#pragma unroll
            for (int r = 0; r < NR; ++r) acc[r][0] = row_dot<C>(st[j].ch[r], st[j].sc[r], xv, xsum, acc[r][0]);
            __builtin_amdgcn_sched_barrier(0);
        } else {
            float xsv[SM];
#pragma unroll
            for (int t = 0; t < SM; ++t) xsv[t] = XSUM ? xsums[t * NCH + cu] : 0.f;
            step_compute_lds<C, NR, SM, true, XSUM>(st[j], (lfloats)xs, xl, cu, acc, xsv);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    float out = 0.f, outu = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int s = 0; s < SM; ++s) {
            const float t = wave_sum(acc[r][s]);
            const float tu = GU ? wave_sum(acc[R + r][s]) : 0.f;
            if (lane == r * SM + s) { out = t; outu = tu; }
        }
    const int r = lane / SM, s = lane % SM;
    if (lane < R * SM && row0 + r < m.O && s < S) epi(s, row0 + r, out, outu);
}

template <int C, int SM, bool GU, int NS, int W, int R>
__global__ void __launch_bounds__(WAVE * W) k_rows_x(MatDev m0, MatDev m1, const float *__restrict__ x, int S,
                                                     float *__restrict__ y, float L) {
    rows_x_body<C, SM, GU, NS, W, R, SM == 1>(m0, m1, x, S, [&](int s, int row, float v, float vu) {
        y[(size_t)s * m0.O + row] = GU ? swiglu(v, vu, L) : v;
    });
}

// ---------------------------------------------------------------------------
// dqg_dequant: out[o][k] = value * scale with value = (decoded - OFFS) *
// VMUL exactly, then one rounding.  One thread per chunk.
// ---------------------------------------------------------------------------
template <int C>
__global__ void __launch_bounds__(256) k_dequant(MatDev m, float *__restrict__ out) {
    using Cd = Codec<C>;
    const int nch = m.K / Cd::CW;
    const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (size_t)m.O * nch) return;
    const int row = (int)(idx / nch), c = (int)(idx % nch);
    const GRow rp = lane_row_ptrs(m, row);
    const typename Cd::Chunk ch = Cd::load(rp, (uint32_t)c);
    const float sc = Cd::SCALED ? ldf(rp.s, (uint32_t)c >> m.shift) : 1.f;
    float *o = out + (size_t)row * m.K + (size_t)c * Cd::CW;
#pragma unroll
    for (int u = 0; u < Cd::UNITS; ++u) {
        float v[Cd::UW];
        if constexpr (Cd::WIDE) {
            float d[Cd::UW];
            Cd::decode_f(ch, u, d);
#pragma unroll
            for (int i = 0; i < Cd::UW; ++i) {
                float t = d[i];   // formats without offset, power or scale pass their values through
                if constexpr (Cd::OFFS != 0.f) t -= Cd::OFFS;
                if constexpr (Cd::VMUL != 1.f) t *= Cd::VMUL;
                if constexpr (Cd::SCALED) t *= sc;
                v[Cd::IDX[i]] = t;
            }
        } else {
            uint32_t pr[Cd::UW / 2];
            Cd::decode(ch, u, pr);
#pragma unroll
            for (int q = 0; q < Cd::UW / 2; ++q) {
                const half2_t h = __builtin_bit_cast(half2_t, pr[q]);
                v[Cd::IDX[2 * q]] = (((float)h.x - Cd::OFFS) * Cd::VMUL) * sc;
                v[Cd::IDX[2 * q + 1]] = (((float)h.y - Cd::OFFS) * Cd::VMUL) * sc;
            }
        }
#pragma unroll
        for (int i = 0; i < Cd::UW; i += 4)
            *reinterpret_cast<float4 *>(o + u * Cd::UW + i) = make_float4(v[i], v[i + 1], v[i + 2], v[i + 3]);
    }
}

// ---------------------------------------------------------------------------
// Routed expert group.
//
// Units: routed slot q = t*k + r (q < S*k) and, with a shared expert, the
// gate/up launch's unit S*k (which serves every token's shared slot) or the
// down launch's units S*k + t (token t's shared slot each).  A routed unit
// whose expert appears at an earlier slot is skipped; the first slot of an
// expert (its owner) serves every slot that names it, one after another, so
// each distinct expert's rows come from HBM once per call.  Slot lists come
// from wave ballots over ids; no host round trip.
// ---------------------------------------------------------------------------
struct SlotBatch {
    int slot;       // the h row it fills: t*k + r for token t's rank r, S*k + t for its shared expert
    int token;
};

// Is unit q the first slot naming expert e?  (wave-uniform)
__device__ __forceinline__ bool owns(const int32_t *ids, int q, int e) {
    const int lane = threadIdx.x & (WAVE - 1);
    for (int base = 0; base < q; base += WAVE) {
        const int i = base + lane;
        const bool hit = i < q && ids[i] == e;
        if (__ballot(hit)) return false;
    }
    return true;
}

// Calls f(batch) for each (slot, token) that uses unit q's expert e, one at
// a time: every slot >= q naming e, or every token's shared slot.
template <typename F>
__device__ __forceinline__ void for_slots(const GroupArgs &a, int q, int e, F &&f) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int nr = a.S * a.k;
    if (q >= nr) {   // shared expert: token t's slot is nr + t
        for (int t = 0; t < a.S; ++t) f(SlotBatch{nr + t, t});
        return;
    }
    for (int base = q; base < nr; base += WAVE) {
        const int i = base + lane;
        uint64_t mask = __ballot(i < nr && a.ids[i] == e);
        while (mask) {
            const int slot = base + __builtin_ctzll(mask);
            mask &= mask - 1;
            f(SlotBatch{slot, slot / a.k});
        }
    }
}

// Copies the batch's token row of x into the block's LDS (all threads).
// Each thread issues up to 8 loads before its first LDS write, so the copy
// costs one round trip per 8 loads, not one per load.
template <int CW>
__device__ __forceinline__ void stage_x(const GroupArgs &a, const SlotBatch &b, lfloats_w xs, bool sums = false) {
    constexpr int U = 8;
    constexpr uint32_t NT = WAVE * WPB_A;   // the gate/up launch's block size
    __syncthreads();   // the previous batch's readers are done
    const uint32_t n4 = a.H / 4;
    const GLOBAL f32x4 *src = (const GLOBAL f32x4 *)(gf(a.x) + (size_t)b.token * a.H);
    for (uint32_t i0 = threadIdx.x; i0 < n4; i0 += U * NT) {
        f32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (i0 + u * NT < n4) v[u] = src[i0 + u * NT];
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (i0 + u * NT < n4) *(LDS f32x4 *)(xs + x_lds_at<CW, GROUP_XPAD>(4 * (i0 + u * NT))) = v[u];
    }
    __syncthreads();
    if (sums) {
        // the sum of each chunk of x, in input order, after the row
        lfloats_w xsum = xs + x_lds_len<CW, GROUP_XPAD>(a.H);
        for (int t = threadIdx.x; t < a.H / CW; t += (int)NT) {
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < CW / 4; ++i) {
                const f32x4 v = *(const LDS f32x4 *)(xs + x_lds_at<CW, GROUP_XPAD>((uint32_t)(t * CW + 4 * i)));
                acc += v.x;
                acc += v.y;
                acc += v.z;
                acc += v.w;
            }
            xsum[t] = acc;
        }
        __syncthreads();
    }
}

// The experts' activation of one slot's gate and up outputs, as the gate/up
// launch writes it to h.
__device__ __forceinline__ float group_act(const GroupArgs &a, int slot, float gv, float uv) {
    if (a.act == ACT_SWIGLU_V4) {   // bf16 gate and up; the weighted activation to bf16
        const float wr = slot < a.S * a.k ? a.w[slot] : 1.f;
        return round_bf16(swiglu(round_bf16(gv), round_bf16(uv), a.limit) * wr);
    }
    return swiglu(gv, uv, a.limit);
}

// gate_up of R rows (row0..) of expert e for one slot, x from LDS.  The
// first chunk's weights are requested before x is staged.
template <int C, int R>
__device__ __forceinline__ void group_gu_batch(const GroupArgs &a, const ExpertDev &ex, int row0,
                                               const SlotBatch &b, lfloats_w xs) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int nch = ex.gate.K / Codec<C>::CW;
    GRow rows[2 * R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        rows[r] = row_ptrs(ex.gate, min(row0 + r, a.I - 1));
        rows[R + r] = row_ptrs(ex.up, min(row0 + r, a.I - 1));
    }
    float acc[2 * R][1];
    Step<C, 2 * R, 1> st;
    const bool have = lane < nch;
    if (have) step_load_w(st, rows, ex.gate.shift, opaque((uint32_t)lane));
    constexpr bool sums = gu1_pairs<C, 2 * R>() && Codec<C>::OFFS != 0.f;
    stage_x<Codec<C>::CW>(a, b, xs, sums);
    dot_rows_lds1<C, 2 * R>(st, have, rows, nch, ex.gate.shift, xs, xs + x_lds_len<Codec<C>::CW, GROUP_XPAD>(a.H),
                            acc);
    float gv = 0.f, uv = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float tg = wave_sum(acc[r][0]);
        const float tu = wave_sum(acc[R + r][0]);
        if (lane == r) { gv = tg; uv = tu; }
    }
    if (lane < R && row0 + lane < a.I) a.h[(size_t)b.slot * a.I + row0 + lane] = group_act(a, b.slot, gv, uv);
}

// Kernel A: grid (row blocks of I, units).  Clears the error flag.  The
// block stages each slot's x row in LDS once; its waves read their slices
// from there.  Every wave of a block stays to the end (block barriers),
// with rows past I clamped and their outputs dropped.
template <int C, int R>
__device__ __forceinline__ void group_gate_up(const GroupArgs &a) {
    extern __shared__ float x_lds_raw[];
    lfloats_w xs = (lfloats_w)x_lds_raw;
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *a.flag = 0;
    // the shared expert's blocks (row y = 0) go first: with several tokens
    // it serves a slot per token, and started last it would set the tail
    const int q = a.shared >= 0 ? (blockIdx.y == 0 ? (int)gridDim.y - 1 : (int)blockIdx.y - 1) : (int)blockIdx.y;
    const int nr = a.S * a.k;
    const int e = __builtin_amdgcn_readfirstlane(q < nr ? a.ids[q] : a.shared);
    if (e < 0 || e >= a.n_experts) return;         // reported by kernel B
    if (q < nr && !owns(a.ids, q, e)) return;
    const int wave = blockIdx.x * (blockDim.x / WAVE) + wave_id();
    const int row0 = wave * R;   // rows past I are clamped in row_ptrs, outputs dropped
    const ExpertDev &ex = a.table[e];
    for_slots(a, q, e, [&](const SlotBatch &b) { group_gu_batch<C, R>(a, ex, row0, b, xs); });
}

template <int C, int R>
__global__ void __launch_bounds__(WAVE * WPB_A) k_group_gate_up(GroupArgs a) { group_gate_up<C, R>(a); }

// The same with a register budget of 5 waves per SIMD (every codec but
// int3), so that a one-token 9-unit group (1152 blocks of 4 waves) is
// resident in one round on 256 CUs.
template <int C, int R>
__global__ void __launch_bounds__(WAVE * WPB_A) __attribute__((amdgpu_waves_per_eu(5)))
k_group_gate_up1(GroupArgs a) { group_gate_up<C, R>(a); }

// down rows row0.. of expert e applied to one slot's h -> d (LDS)
template <int C, int R>
__device__ __forceinline__ void group_down_batch(const GroupArgs &a, const ExpertDev &ex, int row0,
                                                 const SlotBatch &b, float *d) {
    const int lane = threadIdx.x & (WAVE - 1);
    GRow rows[R];
#pragma unroll
    for (int r = 0; r < R; ++r) rows[r] = row_ptrs(ex.down, min(row0 + r, a.H - 1));
    const XGlobal xp[1] = {{gf(a.h + (size_t)b.slot * a.I)}};
    float acc[R][1];
    dot_rows<C, R, 1>(rows, ex.down.K / Codec<C>::CW, ex.down.shift, xp, acc);
    float out = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float t = wave_sum(acc[r][0]);
        if (lane == r) out = t;
    }
    if (lane < R) d[b.slot * R + lane] = a.act == ACT_SWIGLU_V4 ? round_bf16(out) : out;
}

template <int R>
__device__ __forceinline__ void group_combine(const GroupArgs &a, float *d, int row0);

// Kernel B: one block per R rows of H.  Waves take the units from a block
// counter; each unit's outputs go to LDS d[slot][R]; then y[t][row] =
// sum_r w[t][r] * d[t*k+r] in rank order, plus the shared slot.  Sets the
// flag for a bad id.
// Block size: one wave per unit, at most 8 waves (2 per SIMD, so that two
// blocks share a CU; blocks of 9 or more waves were measured to hold one).
constexpr int DOWN_MAX_WAVES = 8;

template <int C, int R>
__device__ __forceinline__ void group_down(const GroupArgs &a) {
    extern __shared__ float d[];
    __shared__ int next_unit;   // the block's next unit that no wave has taken
    const int row0 = blockIdx.x * R;
    const int nr = a.S * a.k;
    // units: the routed slots (each expert once, by its first slot), then
    // each token's shared slot on its own, so that the shared expert's S
    // slots spread over the waves instead of one wave's serial passes
    const int nunits = nr + (a.shared >= 0 ? a.S : 0);
    const int nw = blockDim.x / WAVE;
    const int lane = threadIdx.x & (WAVE - 1);
    if (threadIdx.x == 0) next_unit = nw;
    __syncthreads();
    // wave w starts with unit w, then takes the next untaken one: an
    // expert named by several slots costs its owner a pass per slot and its
    // other slots nothing, so units dealt in turn left some waves more
    // passes than others (measured on MI355X, interleaved: the MXFP4 group
    // at 8 tokens, down 144.5-146.0 -> 132.2-134.3 us; the int4-g32 group at
    // 4 tokens 63.9-64.4 -> 60.9-61.2 us, at 2 34.9-35.8 -> 33.1-34.2 us)
    for (int q = wave_id(); q < nunits;) {
        const int e = __builtin_amdgcn_readfirstlane(q < nr ? a.ids[q] : a.shared);
        if (e < 0 || e >= a.n_experts) {
            if (lane < R) d[q * R + lane] = __int_as_float(0x7FC00000);   // quiet NaN
            if (lane == 0) *a.flag = 1;
        } else if (q >= nr) {   // token q - nr's shared slot
            group_down_batch<C, R>(a, a.table[e], row0, SlotBatch{q, q - nr}, d);
        } else if (owns(a.ids, q, e)) {
            const ExpertDev &ex = a.table[e];
            for_slots(a, q, e, [&](const SlotBatch &b) { group_down_batch<C, R>(a, ex, row0, b, d); });
        }
        int t = 0;
        if (lane == 0) t = atomicAdd(&next_unit, 1);
        q = __builtin_amdgcn_readfirstlane(t);
    }
    group_combine<R>(a, d, row0);
}

// The end of kernel B, after every slot's outputs for rows row0..row0+R-1
// are in d[slot][R] (LDS): y[t][row] = sum_r w[t][r] * d[t*k+r] in rank
// order, plus the shared slot; DeepSeek V4's weights were applied before
// down and its slots are summed in (expert id, rank) order.  All threads.
template <int R>
__device__ __forceinline__ void group_combine(const GroupArgs &a, float *d, int row0) {
    const int nr = a.S * a.k;
    // DeepSeek V4's combine order, after the slots' outputs in LDS: each
    // routed slot's place among its token's (expert id, rank) pairs
    const bool v4 = a.act == ACT_SWIGLU_V4;
    int *sid = reinterpret_cast<int *>(d + (size_t)(nr + (a.shared >= 0 ? a.S : 0)) * R), *ord = sid + nr;
    if (v4)
        for (int q = threadIdx.x; q < nr; q += blockDim.x) sid[q] = a.ids[q];
    __syncthreads();
    if (v4) {
        for (int q = threadIdx.x; q < nr; q += blockDim.x) {
            const int t = q / a.k, rk = q - t * a.k, id = sid[q];
            int pos = 0;
            for (int j = 0; j < a.k; ++j) {
                const int o = sid[t * a.k + j];
                pos += o < id || (o == id && j < rk);
            }
            ord[t * a.k + pos] = rk;
        }
        __syncthreads();
    }
    for (int j = threadIdx.x; j < a.S * R; j += blockDim.x) {
        const int t = j / R, r = j % R;
        if (row0 + r >= a.H) continue;
        float acc = 0.f;
        if (v4) {   // the weights were applied before down
            for (int n = 0; n < a.k; ++n) acc += d[(t * a.k + ord[t * a.k + n]) * R + r];
        } else {
            for (int rk = 0; rk < a.k; ++rk) acc = fmaf(a.w[t * a.k + rk], d[(t * a.k + rk) * R + r], acc);
        }
        if (a.shared >= 0) acc += d[(nr + t) * R + r];
        a.y[(size_t)t * a.H + row0 + r] = acc;
    }
}

// (a budget of 4 waves per SIMD, so that two 8-wave blocks share a CU; int3,
// whose rows of 64-input chunks take more registers, has none)
template <int C, int R>
__global__ void __launch_bounds__(WAVE * DOWN_MAX_WAVES) __attribute__((amdgpu_waves_per_eu(C == C_I3 ? 1 : 4)))
k_group_down(GroupArgs a) { group_down<C, R>(a); }

// One token routed to one expert, no shared expert (a single expert MLP):
// the group's two launches on k_rows_x's block shape, whose blocks fill the
// chip where one unit's group blocks (I/16 of them) leave most CUs idle.
// The per-row arithmetic, the activation and the combine (the one slot's
// weight times its output, or with DeepSeek V4's activation 0 plus the
// output rounded to bf16) are the group kernels', so the bits are theirs.
template <int C, int NS, int W, int R>
__global__ void __launch_bounds__(WAVE * W) k_unit_gate_up(GroupArgs a) {
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.flag = 0;
    const int e = __builtin_amdgcn_readfirstlane(a.ids[0]);
    if (e < 0 || e >= a.n_experts) return;   // reported by the down launch
    const MatDev g = a.table[e].gate, u = a.table[e].up;
    rows_x_body<C, 1, true, NS, W, R, false>(g, u, a.x, 1,
                                      [&](int, int row, float gv, float uv) { a.h[row] = group_act(a, 0, gv, uv); });
}

template <int C, int NS, int W, int R>
__global__ void __launch_bounds__(WAVE * W) k_unit_down(GroupArgs a) {
    const int e = __builtin_amdgcn_readfirstlane(a.ids[0]);
    if (e < 0 || e >= a.n_experts) {   // NaN outputs, and the call reports the id
        const int row = blockIdx.x * W * R + (int)threadIdx.x;
        if ((int)threadIdx.x < W * R && row < a.H) a.y[row] = __int_as_float(0x7FC00000);
        if (threadIdx.x == 0) *a.flag = 1;
        return;
    }
    const MatDev d = a.table[e].down;
    const float w0 = a.w[0];
    const bool v4 = a.act == ACT_SWIGLU_V4;
    rows_x_body<C, 1, false, NS, W, R, false>(d, d, a.h, 1, [&](int, int row, float v, float) {
        a.y[row] = v4 ? 0.f + round_bf16(v) : fmaf(w0, v, 0.f);
    });
}

// Kernel B for one token with a shared expert and 6 to 8 routed ones (a
// decode step), on blocks of R = 24 rows and 2k waves: waves 2r and 2r + 1
// compute the first and second 12 rows of routed rank r, and the shared
// expert's R rows are dealt over the waves (row j to wave j % W, at most
// SPLIT_NX a wave), so that no wave streams a second unit after its first.
// The h of every slot (the k ranks, then the shared slot) is staged once per
// block in LDS, its loads (SPLIT_HN 16-byte loads a thread, clamped
// duplicates writing the same value twice) issued ahead of the weights, so
// that a block reads h from L2 once for 24 rows (measured on MI355X, int4-g32
// group at one token: 17.1-17.2 us against 18.1-18.3 with one wave a rank on
// 12-row blocks, each wave reading its rank's h from L2).  A wave's rows go
// through a ring of SPLIT_DEPTH rows in flight, each row computed as it
// lands.  The per-row arithmetic is step_compute's, so the bits are those of
// k_group_down.  The launcher checks: S == 1, shared >= 0, k in [6, 8], and
// I of 64 chunks (one a lane; I = 2048 for the 32-value chunks of int4 and
// MXFP4).
constexpr int SPLIT_NX = 2, SPLIT_R = 24, SPLIT_HN = 5;
// Rows a wave keeps in flight (measured on MI355X for the int4-g32 group at
// one token, interleaved: depth 2, 3, 4, 6, 8, 10 -> 15.4-15.5, 15.5-15.7,
// 15.2-15.7, 16.4-16.7, 17.7-18.0, 19.2 us; with 16 waves a CU, 4 rows a wave
// keep enough bytes in flight, and fewer rows land in the wave's last stretch).
constexpr int SPLIT_DEPTH = 4;

template <int C>
__global__ void __launch_bounds__(WAVE * 16) __attribute__((amdgpu_waves_per_eu(4)))
k_group_down_split(GroupArgs a) {
    using Cd = Codec<C>;
    constexpr int NX = SPLIT_NX, R = SPLIT_R, RW = R / 2, HN = SPLIT_HN;
    extern __shared__ float lds[];
    const int nr = a.k;            // one token: slot q is rank q, the shared slot is nr
    // LDS: h of slots 0..nr (unpadded), then the slots' outputs d[slot][R]
    lfloats_w hl = (lfloats_w)lds;
    float *d = lds + (size_t)(nr + 1) * a.I;
    const int W = blockDim.x / WAVE, w = wave_id(), lane = threadIdx.x & (WAVE - 1);
    const int rank = w / 2, part = w % 2;
    const int row0 = blockIdx.x * R;
    const uint32_t n4 = (uint32_t)((nr + 1) * a.I / 4), nt = blockDim.x;
    const GLOBAL f32x4 *hsrc = (const GLOBAL f32x4 *)gf(a.h);
    f32x4 hv[HN];
#pragma unroll
    for (int u = 0; u < HN; ++u) hv[u] = hsrc[min((uint32_t)threadIdx.x + u * nt, n4 - 1)];
    const int e = __builtin_amdgcn_readfirstlane(a.ids[rank]);
    const bool ok = e >= 0 && e < a.n_experts;
    const ExpertDev &ex = a.table[ok ? e : a.shared];   // a bad id reads the shared expert, then writes NaN
    const ExpertDev &exs = a.table[a.shared];
    // the wave's rows in order: RW of its rank, then NX of the shared expert
    constexpr int NT = RW + NX, D = SPLIT_DEPTH;
    GRow rows[NT];
#pragma unroll
    for (int r = 0; r < RW; ++r) rows[r] = row_ptrs(ex.down, min(row0 + part * RW + r, a.H - 1));
#pragma unroll
    for (int j = 0; j < NX; ++j) rows[RW + j] = row_ptrs(exs.down, min(row0 + min(w + j * W, R - 1), a.H - 1));
    const int shift = ex.down.shift;
    const uint32_t c = opaque((uint32_t)lane);   // one chunk a lane
    const uint32_t si = c >> shift;
    float out = 0.f;   // lane r: row r's sum
    typename Cd::Chunk ch[D];
    float sc[D];
    // then a ring of D rows in flight: row i's codes and scale are issued
    // when row i - D has been computed
    float xv[Cd::CW];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < D; ++i) {
        ch[i] = Cd::load(rows[i], c);
        sc[i] = Cd::SCALED ? ld_scale(rows[i].s, si) : 1.f;
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int u = 0; u < HN; ++u) {
        const uint32_t i = min((uint32_t)threadIdx.x + u * nt, n4 - 1);
        *(LDS f32x4 *)(hl + 4 * i) = hv[u];
    }
    // x of a slot from the block's LDS copy, and its chunk sum
    const auto x_from_lds = [&](int slot_in_lds) {
#pragma unroll
        for (int q = 0; q < Cd::CW / 4; ++q) {
            const f32x4 t = *(const LDS f32x4 *)(hl + (size_t)slot_in_lds * a.I + c * Cd::CW + 4 * q);
            xv[4 * q] = t.x; xv[4 * q + 1] = t.y; xv[4 * q + 2] = t.z; xv[4 * q + 3] = t.w;
        }
    };
    __syncthreads();   // h staged
    x_from_lds(rank);
    float xs = 0.f;
    if (Cd::OFFS != 0.f) {
#pragma unroll
        for (int i = 0; i < Cd::CW; ++i) xs += xv[i];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        if (i == RW) {
            // the shared rows
            x_from_lds(nr);
            xs = 0.f;
            if (Cd::OFFS != 0.f) {
#pragma unroll
                for (int q = 0; q < Cd::CW; ++q) xs += xv[q];
            }
        }
        const float acc = row_dot<C>(ch[i % D], sc[i % D], xv, xs, 0.f);
        if (i + D < NT) {
            ch[i % D] = Cd::load(rows[i + D], c);
            sc[i % D] = Cd::SCALED ? ld_scale(rows[i + D].s, si) : 1.f;
        }
        // the row's sum over the wave right away, so that only the last
        // rows' reductions remain after the last bytes land
        const float t = wave_sum(acc);
        if (lane == i) out = t;
        __builtin_amdgcn_sched_barrier(0);
    }
    const bool v4 = a.act == ACT_SWIGLU_V4;
    if (lane < RW) d[rank * R + part * RW + lane] = ok ? (v4 ? round_bf16(out) : out) : __int_as_float(0x7FC00000);
    if (lane >= RW && lane < RW + NX) {
        const int xr = w + (lane - RW) * W;
        if (xr < R) d[nr * R + xr] = v4 ? round_bf16(out) : out;
    }
    if (!ok && lane == 0) *a.flag = 1;
    group_combine<R>(a, d, row0);
}

// DeepSeek V4's pass between the activation and down: every block of 128
// consecutive values of a slot's h becomes E4M3 values times the block's
// power-of-two scale.  One wave per block; lane l holds values l and l + 64.
// Multiplying by 2^-j and by 2^j is exact while E4M3's quantum 2^-9 times 2^j
// stays on f32's grid (j >= -140: a block whose largest magnitude is at least
// about 2^-131).
__global__ void __launch_bounds__(256) k_group_act_v4(float *__restrict__ h, int nblk) {
    const int blk = blockIdx.x * 4 + wave_id();
    if (blk >= nblk) return;
    const int lane = threadIdx.x & (WAVE - 1);
    float *p = h + (size_t)blk * 128;
    const float v0 = p[lane], v1 = p[lane + 64];
    const int j = v4_scale_exp(wave_max(fmaxf(fabsf(v0), fabsf(v1))));
    p[lane] = ldexpf(round_e4m3(ldexpf(v0, -j)), j);
    p[lane + 64] = ldexpf(round_e4m3(ldexpf(v1, -j)), j);
}

// ---------------------------------------------------------------------------
// Prefill GEMM on the matrix cores, for batches of several tokens
// ("colibri -- Vulkan backend (docs/vulkan.md)", tier properties: a batch of
// 16 or more rows per expert goes to a tiled GEMM): Y[s][o] = W[o] . x[s],
// and gate_up's h = silu(G x) * (U x).
//
// v_mfma_f32_16x16x32_f16 computes D (16 rows x 16 tokens, f32) from
// A (16 rows x 32 inputs, f16) and B (32 inputs x 16 tokens, f16).  Lane
// layout: A lane l holds row l%16, inputs 8(l/16)..+8 of the window; B lane
// l holds token l%16, the same inputs; D lane l holds rows 4(l/16)..+4 of
// token l%16.  A is the code's value as an f16: the decoded pattern, less
// the code offset for the offset formats (both exact: the values are
// integer multiples of 2^-24, and the matrix cores keep f16 subnormals).
// B is x' = x * 2^-e split as f16 hi + lo, with e per token and 32-input
// window so that x' fits f16, which leaves x' - hi - lo below 2^-22 |x'|.
// A window never crosses a scale group, so each window's D is scaled on the
// vector unit:  acc += (scale * VMUL * 2^e) * D.
// A block is 4 waves; a wave holds 2 row tiles (32 rows of W, or 16 rows of
// G and the same 16 of U) for NC token tiles of 16.  x' for 16 NC tokens x
// GK inputs is staged in LDS per k-step, in the order the decode emits.
// ---------------------------------------------------------------------------
typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));

// Codes of 8 consecutive inputs of one row (a quarter window) and their
// decode into the 4 f16 pairs of an MFMA A operand; PERM[p] is the input
// (0..7) that half p of the operand multiplies.
template <int C>
struct GemmCodec;

//
// The f16 operand of a code: the integer codes as f16 subnormals (a
// non-negative integer n below 1024 in the low bits of an f16 is n * 2^-24),
// an e2m1 code with its magnitude bits at f16 bits 9..11 and its sign at bit
// 15 as e2m1 * 2^-14 (the two formats put the implicit one and the exponent
// bias in the same places), E4M3 and f16 as their values.  So a code's
// value is (operand - OFFS) * VMUL, VMUL a power of two folded into the
// window's scale.

template <>
struct GemmCodec<C_I4> {
    static constexpr int PERM[8] = {0, 4, 1, 5, 2, 6, 3, 7};
    static constexpr float VMUL = Codec<C_I4>::VMUL, OFFS = Codec<C_I4>::OFFS;
    using Raw = uint32_t;
    __device__ static Raw load(gbytes row, uint32_t k) { return *(const GLOBAL uint32_t *)(row + k / 2); }
    __device__ static void decode(Raw w, uint32_t (&pr)[4]) {
        Codec<C_I4>::decode({{w, 0u, 0u, 0u}}, 0, pr);
    }
};

// MXFP4: the f16 high byte of code c is ((c & 7) << 1) | ((c & 8) << 4); it
// is built for the four even and four odd codes of a word at once, then
// v_perm pairs each even code with the next odd one over zero low bytes.
template <>
struct GemmCodec<C_FP4> {
    static constexpr int PERM[8] = {0, 1, 2, 3, 4, 5, 6, 7};
    static constexpr float VMUL = 16384.f, OFFS = 0.f;
    using Raw = uint32_t;
    __device__ static Raw load(gbytes row, uint32_t k) { return *(const GLOBAL uint32_t *)(row + k / 2); }
    __device__ static void decode(Raw w, uint32_t (&pr)[4]) {
        const uint32_t he = ((w << 1) & 0x0E0E0E0Eu) | ((w << 4) & 0x80808080u);   // codes 0,2,4,6
        const uint32_t ho = ((w >> 3) & 0x0E0E0E0Eu) | (w & 0x80808080u);          // codes 1,3,5,7
        pr[0] = __builtin_amdgcn_perm(ho, he, 0x040C000Cu);
        pr[1] = __builtin_amdgcn_perm(ho, he, 0x050C010Cu);
        pr[2] = __builtin_amdgcn_perm(ho, he, 0x060C020Cu);
        pr[3] = __builtin_amdgcn_perm(ho, he, 0x070C030Cu);
    }
};

// int8: q ^ 0x80 = q + 128 as an unsigned byte; v_perm drops bytes into the
// low byte of each f16 half.
template <>
struct GemmCodec<C_I8> {
    static constexpr int PERM[8] = {0, 2, 1, 3, 4, 6, 5, 7};
    static constexpr float VMUL = 16777216.f, OFFS = 128.f / 16777216.f;
    using Raw = u32x2;
    __device__ static Raw load(gbytes row, uint32_t k) { return *(const GLOBAL u32x2 *)(row + k); }
    __device__ static void decode(Raw w, uint32_t (&pr)[4]) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t b = (j ? w.y : w.x) ^ 0x80808080u;
            pr[2 * j] = __builtin_amdgcn_perm(0u, b, 0x0C020C00u);       // inputs 0, 2
            pr[2 * j + 1] = __builtin_amdgcn_perm(0u, b, 0x0C030C01u);   // inputs 1, 3
        }
    }
};

// E4M3 -> f32 -> f16 pairs: every E4M3 value is an f16, so both steps are exact.
template <>
struct GemmCodec<C_FP8> {
    static constexpr int PERM[8] = {0, 1, 2, 3, 4, 5, 6, 7};
    static constexpr float VMUL = 1.f, OFFS = 0.f;
    using Raw = u32x2;
    __device__ static Raw load(gbytes row, uint32_t k) { return *(const GLOBAL u32x2 *)(row + k); }
    __device__ static void decode(Raw w, uint32_t (&pr)[4]) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t v = j ? w.y : w.x;
            const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(v, false);
            const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(v, true);
            pr[2 * j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a.x, a.y));
            pr[2 * j + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(b.x, b.y));
        }
    }
};

// f16 rows: the 16 bytes of 8 inputs are the operand as they stand.
template <>
struct GemmCodec<C_F16> {
    static constexpr int PERM[8] = {0, 1, 2, 3, 4, 5, 6, 7};
    static constexpr float VMUL = 1.f, OFFS = 0.f;
    using Raw = u32x4;
    __device__ static Raw load(gbytes row, uint32_t k) { return *(const GLOBAL u32x4 *)(row + 2 * k); }
    __device__ static void decode(Raw w, uint32_t (&pr)[4]) {
        pr[0] = w.x; pr[1] = w.y; pr[2] = w.z; pr[3] = w.w;
    }
};

// A k-step is GK(NC) inputs: 512 for one token tile, 256 for two, 128 for
// four, so that the staged x' (16 NC tokens x GK, hi and lo) stays near
// 34 KB and batches of few tokens take few, long steps (each step exposes one
// memory latency).
template <int NC>
constexpr int gemm_k() { return 512 / NC; }
constexpr int GROWS = 128;         // row slots per block: 4 waves x 2 tiles x 16
// The sum over K is taken per chunk of GEMM_KC inputs (a whole number of
// k-steps for every NC), and the chunk sums are added in chunk order from
// 0.  A block either walks all chunks itself or, when the grid would be too
// small to fill the chip, computes one chunk into a workspace that
// k_gemm_reduce adds up in the same order: the bits are the same either way.
constexpr int GEMM_KC = 512;

// 16-byte aligned so that the operand reads and the staging writes are
// single ds_read_b128 / ds_write_b128 (with 4-byte alignment the compiler
// splits each into dword pairs, twice the LDS instructions, and dword
// accesses at the operand's row stride collide in the banks).
template <int NC>
struct alignas(16) GemmLds {
    static constexpr int GK = gemm_k<NC>(), GWIN = GK / 32, GT = 16 * NC, XS = GK + 8;   // XS padded
    _Float16 xh[GT][XS];
    _Float16 xl[GT][XS];
    float xe[GT][GWIN];    // 2^e of the token for each window
    float sc[GWIN][GROWS]; // scale * VMUL per window and row slot
};

// One 32-input window of a token as the B operand: x' = x * 2^-e with e
// chosen so that max |x'| < 2^15, split as f16 hi + lo, quarter g (8
// inputs) in the decode's order PERM.  Returns 2^e.
template <int C>
__device__ __forceinline__ float split_window(const f32x4 (&v)[8], h16x8 (&hi)[4], h16x8 (&lo)[4]) {
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
    int ex = 0;
    if (mx > 0.f) { frexpf(mx, &ex); ex -= 15; }   // mx * 2^-ex < 2^15
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int i = 8 * g + GemmCodec<C>::PERM[p];
            const float xv = ldexpf(v[i >> 2][i & 3], -ex);
            const _Float16 h = (_Float16)xv;
            hi[g][p] = h;
            lo[g][p] = (_Float16)(xv - (float)h);
        }
    return ldexpf(1.f, ex);
}

// Row of slot (wave w, tile t, lane row r) and the matrix it comes from.
template <bool GU>
__device__ __forceinline__ int gemm_row(int block_row, int w, int t, int r) {
    return GU ? block_row + 16 * w + r : block_row + 32 * w + 16 * t + r;
}

// ws == nullptr: the block sums all of K and writes y (GU: swiglu(g, u)).
// Otherwise the block sums chunk blockIdx.z only and writes the raw sums to
// ws[(z * MATS + mat) * S + s][row] (MATS = 2 for GU, gate then up, else 1;
// rows 0 .. gridDim.x * rows per block - 1 all have a slot, row stride op).
// With 2 or 4 token tiles the LDS tile is double-buffered (one barrier per
// k-step; two blocks still fit a CU); with one it is single (its tile is
// larger).
template <int C, bool GU, int NC>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
k_gemm(MatDev m0, MatDev m1, const float *__restrict__ x, int S, float *__restrict__ y, float limit,
       float *__restrict__ ws, int op) {
    using Gc = GemmCodec<C>;
    using Cd = Codec<C>;
    using Lt = GemmLds<NC>;
    constexpr int GK = Lt::GK, GWIN = Lt::GWIN;
    constexpr int TPT = 256 / Lt::GT;   // staging threads per token, one window each
    static_assert(TPT * 32 == GK, "one staging thread per token and window");
    constexpr bool DB = NC > 1;
    __shared__ Lt Ls[DB ? 2 : 1];
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = wave_id();
    const int O = m0.O, K = m0.K;
    const int block_row = blockIdx.x * (GU ? GROWS / 2 : GROWS);
    const int s0 = blockIdx.y * (16 * NC);
    const int kbeg = ws ? blockIdx.z * GEMM_KC : 0, kend = ws ? min(K, kbeg + GEMM_KC) : K;
    const int lr = lane & 15, lq = lane >> 4;   // A/B: row or token within a tile; quarter of the window
    // this lane's A rows (clamped; rows past O are computed and dropped)
    gbytes arow[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const MatDev &m = (GU && t == 1) ? m1 : m0;
        const int row = min(gemm_row<GU>(block_row, w, t, lr), O - 1);
        arow[t] = (gbytes)(m.q + (size_t)row * m.qstride);
    }
    float acc[2][NC][4], tot[2][NC][4];   // this chunk's sums; the chunk sums so far
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[t][c][i] = tot[t][c][i] = 0.f;

    // Software pipeline over k-steps: the codes, x and scales of step k0 + GK
    // are requested before step k0 is computed, so their latency hides
    // behind the matrix-core work.
    const int tt = tid / TPT, qq = tid % TPT;   // staging: token tt, window qq (32 inputs)
    constexpr int SCN = GWIN * GROWS / 256;     // scales staged per thread
    typename Gc::Raw raw[2][GWIN], raw_n[2][GWIN];
    f32x4 xv_n[8];
    float sc_n[SCN];
    const auto fetch = [&](int k0) {
        const int nwin = min(GWIN, (kend - k0) / 32);   // K is a multiple of 32
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int j = 0; j < GWIN; ++j)
                if (j < nwin) raw_n[t][j] = Gc::load(arow[t], (uint32_t)(k0 + 32 * j + 8 * lq));
        const int s = s0 + tt, kb = k0 + 32 * qq;
        const bool live = s < S && qq < nwin;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            xv_n[i] = live ? *(const GLOBAL f32x4 *)(gf(x) + (size_t)s * K + kb + 4 * i) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int h = 0; h < SCN; ++h) {
            const int i = tid + 256 * h;   // GWIN * GROWS entries
            const int j = i / GROWS, slot = i - j * GROWS;
            const int sw = slot >> 5, st = (slot >> 4) & 1, sr = slot & 15;
            const MatDev &m = (GU && st == 1) ? m1 : m0;
            const int row = min(gemm_row<GU>(block_row, sw, st, sr), O - 1);
            const int k = k0 + 32 * j;
            if constexpr (Cd::SCALED)
                sc_n[h] = j < nwin ? m.s[(size_t)(row >> m.srow) * m.sstride + ((uint32_t)(k / Cd::CW) >> m.shift)] * Gc::VMUL
                                   : 0.f;
            else
                sc_n[h] = Gc::VMUL;
        }
    };
    fetch(kbeg);
    int buf = 0;
    for (int k0 = kbeg; k0 < kend; k0 += GK) {
        Lt &L = Ls[buf];
        const int nwin = min(GWIN, (kend - k0) / 32);
        f32x4 v[8];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int j = 0; j < GWIN; ++j) raw[t][j] = raw_n[t][j];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = xv_n[i];
        // Single buffer: the previous step's readers of L must be done.
        // Double: L was last read two steps ago, before the barrier below
        // of the previous step, which every wave has passed.
        if (!DB) __syncthreads();
        // stage x' of token tt, window qq, scaled by a power of two of its own
        {
            h16x8 hi[4], lo[4];
            const float e2 = split_window<C>(v, hi, lo);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                *(LDS h16x8 *)&L.xh[tt][32 * qq + 8 * g] = hi[g];
                *(LDS h16x8 *)&L.xl[tt][32 * qq + 8 * g] = lo[g];
            }
            L.xe[tt][qq] = e2;
        }
#pragma unroll
        for (int h = 0; h < SCN; ++h) {
            const int i = tid + 256 * h, j = i / GROWS;
            L.sc[j][i - j * GROWS] = sc_n[h];
        }
        __syncthreads();
        if (k0 + GK < kend) fetch(k0 + GK);   // next step's requests go out now
        // the 2^e of every window of this step, for the tokens of this lane's D columns
        float xe[NC][GWIN];
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int q = 0; q < GWIN / 4; ++q) {
                const f32x4 e4 = *(LDS f32x4 *)&L.xe[16 * c + lr][4 * q];
                xe[c][4 * q] = e4.x; xe[c][4 * q + 1] = e4.y; xe[c][4 * q + 2] = e4.z; xe[c][4 * q + 3] = e4.w;
            }
#pragma unroll
        for (int j = 0; j < GWIN; ++j) {
            if (j >= nwin) continue;   // the chunk's last step may hold fewer windows
            h16x8 a[2];
            f32x4 sc4[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                uint32_t pr[4];
                Gc::decode(raw[t][j], pr);
                if constexpr (Gc::OFFS != 0.f) {
                    // offset codes to signed values: exact, the f16 patterns
                    // are integer multiples of 2^-24 far below f16's precision
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const half2_t o = half2_t{(_Float16)(-Gc::OFFS), (_Float16)(-Gc::OFFS)};
                        pr[q] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, pr[q]) + o);
                    }
                }
                a[t] = __builtin_bit_cast(h16x8, u32x4{pr[0], pr[1], pr[2], pr[3]});
                sc4[t] = *(LDS f32x4 *)&L.sc[j][32 * w + 16 * t + 4 * lq];
            }
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int tok = 16 * c + lr;
                const h16x8 bh = *(LDS h16x8 *)&L.xh[tok][32 * j + 8 * lq];
                const h16x8 bl = *(LDS h16x8 *)&L.xl[tok][32 * j + 8 * lq];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    f32x4 d = {0.f, 0.f, 0.f, 0.f};
                    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t], bh, d, 0, 0, 0);
                    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t], bl, d, 0, 0, 0);
                    // the D lanes of token 16c + lane%16 take its window's 2^e
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[t][c][i] = fmaf(sc4[t][i] * xe[c][j], d[i], acc[t][c][i]);
                }
            }
        }
        if ((k0 + GK) % GEMM_KC == 0 || k0 + GK >= kend) {   // a chunk ends with this step
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int c = 0; c < NC; ++c)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        tot[t][c][i] += acc[t][c][i];
                        acc[t][c][i] = 0.f;
                    }
        }
        if (DB) buf ^= 1;
    }
    // D lane layout: rows 4*lq + i of each tile, token 16c + lr
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int s = s0 + 16 * c + lr;
        if (s >= S) continue;
        if (ws) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int row = gemm_row<GU>(block_row, w, GU ? 0 : t, 4 * lq), mat = GU ? t : 0;
                float *p = ws + ((size_t)(blockIdx.z * (GU ? 2 : 1) + mat) * S + s) * op + row;
                *(f32x4 *)p = f32x4{tot[t][c][0], tot[t][c][1], tot[t][c][2], tot[t][c][3]};
            }
            continue;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (GU) {
                const int row = gemm_row<GU>(block_row, w, 0, 4 * lq + i);
                if (row < O) y[(size_t)s * O + row] = swiglu(tot[0][c][i], tot[1][c][i], limit);
            } else {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int row = gemm_row<GU>(block_row, w, t, 4 * lq + i);
                    if (row < O) y[(size_t)s * O + row] = tot[t][c][i];
                }
            }
        }
    }
}

// Sums the chunk partials of k_gemm in chunk order, one output per thread.
template <bool GU>
__global__ void __launch_bounds__(256) k_gemm_reduce(const float *__restrict__ ws, int nch, int S, int O, int op,
                                                     float *__restrict__ y, float limit) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (size_t)S * O) return;
    const int s = (int)(i / O), o = (int)(i - (size_t)s * O);
    const size_t plane = (size_t)S * op;   // one (chunk, matrix) slice
    const float *p = ws + (size_t)s * op + o;
    float g = 0.f, u = 0.f;
    // 8 chunks' loads in flight at a time, added in chunk order
    constexpr int U = 8;
    for (int z0 = 0; z0 < nch; z0 += U) {
        float vg[U], vu[U];
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int z = z0 + i;
            vg[i] = vu[i] = 0.f;
            if (z < nch) {
                vg[i] = p[(size_t)(GU ? 2 * z : z) * plane];
                if (GU) vu[i] = p[(size_t)(2 * z + 1) * plane];
            }
        }
#pragma unroll
        for (int i = 0; i < U; ++i) {
            if (z0 + i < nch) {
                g += vg[i];
                if (GU) u += vu[i];
            }
        }
    }
    y[i] = GU ? swiglu(g, u, limit) : g;
}

// ---------------------------------------------------------------------------
// The GEMM route's split-K chunk for one tile of up to 16 tokens with 4-bit
// codes and one scale per row and 32-input window (int4-g32, MXFP4), shaped
// for batches that stream each weight once.  The products, their order and
// the chunk sums are k_gemm's (same A and B operands in the same lanes,
// the same two matrix-core products a window, the same scaling and order),
// so the bits are its.  A block is 8 waves over one 512-input chunk; a wave
// takes 2 row tiles of 16 (GU: 16 rows of gate and the same 16 of up).
// Every code and scale load of a wave goes out at once, 16 bytes a lane.
// A code load covers 8 rows x 128 bytes (pieces of 64 bytes a row stream
// markedly slower on MI355X): load (p, t, h) gives lane l the 32 codes of
// window 8p + l / 8 of row 8h + l % 8 of tile t.  Three exchanges of a lane
// bit with a register bit (lane bit 5 by v_permlane32_swap, 4 by
// v_permlane16_swap, 3 by a row_ror:8 DPP move and a select) leave lane l
// quarter l / 16 of each window of row l % 16, the A operand's layout.
// x' of the chunk is split once a block.
// ---------------------------------------------------------------------------
constexpr int GV_W = 8;   // waves a block

// Exchanges lane bit 3 with the register pair's index: afterwards a holds
// what lanes with bit 3 clear held in a and b (lane L of b's at L ^ 8), and b
// what lanes with bit 3 set held.  hi8: this lane's bit 3.
__device__ __forceinline__ void swap_lane_bit3(uint32_t &a, uint32_t &b, bool hi8) {
    const uint32_t ra = (uint32_t)__builtin_amdgcn_mov_dpp((int)a, 0x128, 0xF, 0xF, false);   // row_ror:8: lane L ^ 8
    const uint32_t rb = (uint32_t)__builtin_amdgcn_mov_dpp((int)b, 0x128, 0xF, 0xF, false);
    const uint32_t na = hi8 ? rb : a, nb = hi8 ? b : ra;
    a = na;
    b = nb;
}

struct alignas(16) GvLds {
    _Float16 xh[16][GEMM_KC + 8];          // x' hi, token, input (padded rows)
    _Float16 xl[16][GEMM_KC + 8];          // x' lo
    float xe[16][GEMM_KC / 32];            // 2^e of each token and window
    float sc[GV_W][2][GEMM_KC / 32][16];   // per wave and tile: scale * VMUL by window, row
};

template <int C, bool GU>
__global__ void __launch_bounds__(WAVE * GV_W) __attribute__((amdgpu_waves_per_eu(4)))
k_gemv_mma(MatDev m0, MatDev m1, const float *__restrict__ x, int S, float *__restrict__ ws, int op) {
    using Gc = GemmCodec<C>;
    constexpr int GWIN = GEMM_KC / 32;
    static_assert(GWIN == 16, "four loads of 16 bytes a row cover a chunk");
    __shared__ GvLds L;
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = wave_id();
    const int lr = lane & 15, lq = lane >> 4;
    const int O = m0.O, K = m0.K;
    const int block_row = blockIdx.x * (GU ? 16 * GV_W : 32 * GV_W);
    const int kbeg = blockIdx.y * GEMM_KC;
    // x of the chunk, 16 bytes a lane and 1 KiB a load: load i of wave w
    // covers token (4w + i) / 2 (tokens past S repeat the last; their
    // outputs are dropped), 16-byte units 64 ((4w + i) % 2) + lane, so lane
    // l holds inputs 4 (l % 8) .. + 3 of window 8 ((4w + i) % 2) + l / 8
    f32x4 xv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int f = 4 * w + i;
        xv[i] = *(const GLOBAL f32x4 *)(gf(x) + (size_t)min(f >> 1, S - 1) * K + kbeg + 4 * (64 * (f & 1) + lane));
    }
    // this lane's rows for the codes (rows 8h + l % 8 of each tile) and the scales (row lane / 4)
    gbytes arow[2][2];
    gfloats srow[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const MatDev &m = (GU && t == 1) ? m1 : m0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int ra = min(gemm_row<GU>(block_row, w, t, 8 * h + (lane & 7)), O - 1);
            arow[t][h] = (gbytes)(m.q + (size_t)ra * m.qstride);   // per lane: not gb / gf, which take lane 0's
        }
        const int rs = min(gemm_row<GU>(block_row, w, t, lane >> 2), O - 1);
        srow[t] = (gfloats)(m.s + (size_t)rs * m.sstride);
    }
    // stage x' = x 2^-e as f16 hi + lo, e per token and window from the
    // window's largest magnitude (the 8 lanes of a window share it through
    // DPP), each value split as split_window splits it; the two lanes of a
    // quarter swap halves so that one writes its hi and the other its lo,
    // in the decode's order PERM
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int f = 4 * w + i, tok = f >> 1, win = 8 * (f & 1) + (lane >> 3), a = lane & 7;
        const f32x4 v = xv[i];
        float mx = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
        mx = fmaxf(mx, dpp_mov<0xB1>(mx));    // quad_perm [1,0,3,2]
        mx = fmaxf(mx, dpp_mov<0x4E>(mx));    // quad_perm [2,3,0,1]
        mx = fmaxf(mx, dpp_mov<0x141>(mx));   // row_half_mirror: the other quad of the 8
        int ex = 0;
        if (mx > 0.f) { frexpf(mx, &ex); ex -= 15; }   // mx * 2^-ex < 2^15
        _Float16 h[4], l[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float xs = ldexpf(v[e], -ex);
            h[e] = (_Float16)xs;
            l[e] = (_Float16)(xs - (float)h[e]);
        }
        // lane a % 2 == 0 holds inputs 0..3 of quarter a / 2, the other 4..7;
        // the first keeps its hi and takes the other's, the second its lo
        const bool odd = a & 1;
        const uint32_t m0 = __builtin_bit_cast(uint32_t, odd ? half2_t{l[0], l[1]} : half2_t{h[0], h[1]});
        const uint32_t m1 = __builtin_bit_cast(uint32_t, odd ? half2_t{l[2], l[3]} : half2_t{h[2], h[3]});
        const uint32_t s0 = __builtin_bit_cast(uint32_t, odd ? half2_t{h[0], h[1]} : half2_t{l[0], l[1]});
        const uint32_t s1 = __builtin_bit_cast(uint32_t, odd ? half2_t{h[2], h[3]} : half2_t{l[2], l[3]});
        const uint32_t t0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s0, 0xB1, 0xF, 0xF, false);
        const uint32_t t1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s1, 0xB1, 0xF, 0xF, false);
        const half2_t q0[2] = {__builtin_bit_cast(half2_t, odd ? t0 : m0), __builtin_bit_cast(half2_t, odd ? t1 : m1)};
        const half2_t q1[2] = {__builtin_bit_cast(half2_t, odd ? m0 : t0), __builtin_bit_cast(half2_t, odd ? m1 : t1)};
        h16x8 o;
#pragma unroll
        for (int pp = 0; pp < 8; ++pp) {
            const int in = Gc::PERM[pp];   // input of the quarter at position pp
            const half2_t &src = in < 4 ? q0[(in & 3) >> 1] : q1[(in & 3) >> 1];
            o[pp] = (in & 1) ? src.y : src.x;
        }
        _Float16(*dst)[GEMM_KC + 8] = odd ? L.xl : L.xh;
        *(LDS h16x8 *)&dst[tok][32 * win + 8 * (a >> 1)] = o;
        if (a == 0) L.xe[tok][win] = ldexpf(1.f, ex);
    }
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    // then the scales and the codes, in the order the windows use them:
    // requested only now, so that x came back through an idle memory
    // system, and each window's products wait for their own codes while
    // the later ones stream
    f32x4 scv[2];
    u32x4 raw[2][2][2];   // [half of the chunk p][tile t][row half h]
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 2; ++t)
        scv[t] = __builtin_nontemporal_load((const GLOBAL f32x4 *)(srow[t] + kbeg / 32 + 4 * (lane & 3)));
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint4 v = ld16(arow[t][h], (uint32_t)(kbeg / 2 + 128 * p + 16 * (lane >> 3)));
                raw[p][t][h] = u32x4{v.x, v.y, v.z, v.w};
            }
    __builtin_amdgcn_sched_barrier(0);
    // the wave's own scales by window and row (no other wave reads them)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) L.sc[w][t][4 * (lane & 3) + i][lane >> 2] = scv[t][i] * Gc::VMUL;
    float acc[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][i] = 0.f;
    // window j's x operands and scales are read during window j - 1; each
    // window's scaled sums are complete before the next window's reads
    // (left to itself the compiler runs every product first and holds all
    // 32 results, which spills)
    h16x8 bh_n = *(LDS h16x8 *)&L.xh[lr][8 * lq];
    h16x8 bl_n = *(LDS h16x8 *)&L.xl[lr][8 * lq];
    float xe_n = L.xe[lr][0];
    f32x4 sc_n[2] = {*(LDS f32x4 *)&L.sc[w][0][0][4 * lq], *(LDS f32x4 *)&L.sc[w][1][0][4 * lq]};
    uint32_t a32[2][8];   // the A dwords of the 8 windows of a chunk half, by window
    const bool hi8 = (lane >> 3) & 1;
#pragma unroll
    for (int j = 0; j < GWIN; ++j) {
        if (j % 8 == 0) {
            // codes of windows j .. j + 7 to the A layout.  Before: lane
            // (r % 8) + 8 (w % 8) holds row r, window w, in register (row
            // half, quarter).  Swapping lane bit 5 with the quarter's bit 1,
            // lane bit 4 with its bit 0 and lane bit 3 with the row half
            // leaves lane r + 16 q holding quarter q of row r, in register
            // w % 8.
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const u32x4 r0 = raw[j / 8][t][0], r1 = raw[j / 8][t][1];
                const auto h0q0 = __builtin_amdgcn_permlane32_swap(r0.x, r0.z, false, false);   // [window bit 2]
                const auto h0q1 = __builtin_amdgcn_permlane32_swap(r0.y, r0.w, false, false);
                const auto h1q0 = __builtin_amdgcn_permlane32_swap(r1.x, r1.z, false, false);
                const auto h1q1 = __builtin_amdgcn_permlane32_swap(r1.y, r1.w, false, false);
#pragma unroll
                for (int w2 = 0; w2 < 2; ++w2) {
                    const auto u0 = __builtin_amdgcn_permlane16_swap(h0q0[w2], h0q1[w2], false, false);   // [window bit 1]
                    const auto u1 = __builtin_amdgcn_permlane16_swap(h1q0[w2], h1q1[w2], false, false);
#pragma unroll
                    for (int w1 = 0; w1 < 2; ++w1) {
                        uint32_t a = u0[w1], b = u1[w1];
                        swap_lane_bit3(a, b, hi8);   // a: window bit 0 clear, b: set
                        a32[t][4 * w2 + 2 * w1] = a;
                        a32[t][4 * w2 + 2 * w1 + 1] = b;
                    }
                }
            }
        }
        const h16x8 bh = bh_n, bl = bl_n;
        const float xe = xe_n;
        const f32x4 scj[2] = {sc_n[0], sc_n[1]};
        if (j + 1 < GWIN) {
            bh_n = *(LDS h16x8 *)&L.xh[lr][32 * (j + 1) + 8 * lq];
            bl_n = *(LDS h16x8 *)&L.xl[lr][32 * (j + 1) + 8 * lq];
            xe_n = L.xe[lr][j + 1];
            sc_n[0] = *(LDS f32x4 *)&L.sc[w][0][j + 1][4 * lq];
            sc_n[1] = *(LDS f32x4 *)&L.sc[w][1][j + 1][4 * lq];
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            uint32_t pr[4];
            Gc::decode(a32[t][j % 8], pr);
            if constexpr (Gc::OFFS != 0.f) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const half2_t o = half2_t{(_Float16)(-Gc::OFFS), (_Float16)(-Gc::OFFS)};
                    pr[q] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, pr[q]) + o);
                }
            }
            const h16x8 a = __builtin_bit_cast(h16x8, u32x4{pr[0], pr[1], pr[2], pr[3]});
            f32x4 d = {0.f, 0.f, 0.f, 0.f};
            d = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bh, d, 0, 0, 0);
            d = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bl, d, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[t][i] = fmaf(scj[t][i] * xe, d[i], acc[t][i]);
        }
        asm volatile("" : "+v"(acc[0][0]), "+v"(acc[0][1]), "+v"(acc[0][2]), "+v"(acc[0][3]), "+v"(acc[1][0]),
                     "+v"(acc[1][1]), "+v"(acc[1][2]), "+v"(acc[1][3])::"memory");
    }
    // the chunk's sums as k_gemm adds them up from 0; D lane layout: rows
    // 4 lq + i of each tile, token lr
    if (lr < S) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int row = gemm_row<GU>(block_row, w, GU ? 0 : t, 4 * lq), mat = GU ? t : 0;
            float *p = ws + ((size_t)(blockIdx.y * (GU ? 2 : 1) + mat) * S + lr) * op + row;
            *(f32x4 *)p = f32x4{0.f + acc[t][0], 0.f + acc[t][1], 0.f + acc[t][2], 0.f + acc[t][3]};
        }
    }
}

// ---------------------------------------------------------------------------
// Router: logits -> scores -> top-k -> (ids, w), one wave per token.  The
// scores are softmax (max subtracted) or sigmoid; the pick key is the logit
// itself (both scores keep the logits' order) or, with a bias, score +
// bias.  A pick is a wave-wide maximum of (ordered key, inverted index), so
// equal keys go to the lower index; the picked expert's score is its
// weight, renormalised over the k picks on request and scaled.
// ---------------------------------------------------------------------------
// Order-preserving map of a float's bits to an unsigned integer.
__device__ __forceinline__ uint32_t float_order(float f) {
    const uint32_t b = __float_as_uint(f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int m = 1; m < WAVE; m <<= 1) {
        const uint64_t o = __shfl_xor(v, m);
        v = o > v ? o : v;
    }
    return v;
}

constexpr int ROUTE_WAVES = 4;   // tokens per block

template <int NJ>   // experts per lane: E <= 64 * NJ
__global__ void __launch_bounds__(WAVE * ROUTE_WAVES) k_route(RouteArgs a) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int t = blockIdx.x * ROUTE_WAVES + wave_id();
    if (t >= a.S) return;   // the whole wave: t is uniform
    const float *l = a.logits + (size_t)t * a.E;
    float lv[NJ], p[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int e = lane + WAVE * j;
        lv[j] = e < a.E ? l[e] : -INFINITY;
    }
    if (a.mode == 0) {
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < NJ; ++j) mx = fmaxf(mx, lv[j]);
        mx = wave_max(mx);
        float z = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            p[j] = lane + WAVE * j < a.E ? expf(lv[j] - mx) : 0.f;
            z += p[j];
        }
        z = wave_sum(z);
#pragma unroll
        for (int j = 0; j < NJ; ++j) p[j] = p[j] / z;
    } else {
#pragma unroll
        for (int j = 0; j < NJ; ++j) p[j] = lane + WAVE * j < a.E ? 1.f / (1.f + expf(-lv[j])) : 0.f;
    }
    // key: ordered pick value above, 0xFFFFFFFF - e below; 0 = not pickable
    uint64_t key[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int e = lane + WAVE * j;
        if (e < a.E) {
            const float kf = a.bias ? p[j] + a.bias[e] : lv[j];
            key[j] = ((uint64_t)float_order(kf) << 32) | (0xFFFFFFFFu - (uint32_t)e);
        } else {
            key[j] = 0;
        }
    }
    float mine = 0.f, sum = 0.f;
    int my_id = 0;
    for (int r = 0; r < a.k; ++r) {
        uint64_t best = 0;
#pragma unroll
        for (int j = 0; j < NJ; ++j) best = key[j] > best ? key[j] : best;
        best = wave_max_u64(best);
        const int e = (int)(0xFFFFFFFFu - (uint32_t)best);   // uniform
        const int owner = e & (WAVE - 1), jj = e / WAVE;
        float pv = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            if (j == jj) pv = p[j];
            if (j == jj && lane == owner) key[j] = 0;   // taken
        }
        pv = __shfl(pv, owner);
        sum += pv;
        if (lane == r) { mine = pv; my_id = e; }
    }
    if (lane < a.k) {
        const float v = a.renorm ? mine / sum : mine;
        a.ids[(size_t)t * a.k + lane] = my_id;
        a.w[(size_t)t * a.k + lane] = v * a.w_scale;
    }
}

// ---------------------------------------------------------------------------
// dqg_read_bytes: a plain streaming read, the ceiling the weight streams are
// measured against.  Wave w reads 1 KB pieces w, w + W, w + 2W, ... with 16-B
// non-temporal loads, two pieces in flight; blocks of 4 waves, 8 a CU (32 KB
// a CU in flight measured best on MI355X).  The XOR of the bytes goes to
// *sink only if it equals a value no input of a constant fill gives, so
// nothing is written in practice and no load can be dropped.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8)))
k_read(const u32x4 *__restrict__ p, uint64_t npieces, uint32_t *sink) {
    const uint32_t lane = threadIdx.x & (WAVE - 1);
    const uint64_t nw = (uint64_t)gridDim.x * (blockDim.x / WAVE);
    uint64_t k = (uint64_t)blockIdx.x * (blockDim.x / WAVE) + wave_id();
    uint32_t acc = 0;
    for (; k + nw < npieces; k += 2 * nw) {
        const u32x4 a = __builtin_nontemporal_load((const GLOBAL u32x4 *)(p + k * WAVE + lane));
        const u32x4 b = __builtin_nontemporal_load((const GLOBAL u32x4 *)(p + (k + nw) * WAVE + lane));
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w;
    }
    if (k < npieces) {
        const u32x4 a = __builtin_nontemporal_load((const GLOBAL u32x4 *)(p + k * WAVE + lane));
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (acc == 0x9E3779B9u) *sink = acc;
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
constexpr int WPB = 4;   // waves per block for the row kernels

// Launch, with start/stop events attached to the dispatch when timing is on.
template <typename K, typename... Args>
void launch(const char *name, K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t st, Args... args) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (prof_slot(name, &e0, &e1))
        hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, st, e0, e1, 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, lds, st, args...);
}

constexpr int MM_R = 4;   // rows per wave of the general per-row kernel
// Inputs of x per K-chunk: the largest multiple of 64 code chunks that keeps
// SM tokens within 64 KB of LDS, or the whole of K.  (Every format's batch
// size keeps at least 64 code chunks within it: int3's 64-input chunks take
// at most 4 tokens a pass.)
constexpr int MM_LDS_BYTES = 64 * 1024;
template <int C, int SM>
int matmul_kc(int K) {
    const int unit = WAVE * Codec<C>::CW;            // inputs per 64 code chunks
    const int fit = (MM_LDS_BYTES / 4 / SM) / unit * unit;
    return K <= fit ? K : fit;
}

template <int C, int R, int SM>
hipError_t go_matmul(const MatDev &m, const float *x, int S, float *y, hipStream_t st) {
    const int rows_per_block = R * WPB;
    dim3 grid((m.O + rows_per_block - 1) / rows_per_block);
    static_assert(SM * WAVE * Codec<C>::CW * 4 <= MM_LDS_BYTES, "64 code chunks of x per token fit the LDS budget");
    const int KC = matmul_kc<C, SM>(m.K);
    launch("matmul", (k_rows_lds<C, R, SM, false>), grid, dim3(WAVE * WPB),
           (size_t)SM * x_lds_len<Codec<C>::CW>(KC) * 4, st, m, m, x, S, y, KC, INFINITY);
    return hipGetLastError();
}

// The matrix-core GEMM from this many tokens on: where it measured faster
// than the per-row route on MI355X.  The per-row route takes its tokens 8 at
// a time, so 9 to 16 tokens cost it two passes over the weights; the GEMM
// with split-K costs about the same from 8 to 16 tokens.  Kernel times on
// 6144 x 6144: matmul at 8 tokens per row 29-36 us, GEMM 28-37 us (even);
// at 9 tokens per row 54-66 us, GEMM 27-37 us.  gate_up (two such
// matrices) at 8 tokens: int4 53 us per row against 48 GEMM, E4M3 49
// against 41, f16 58 against 51, int8 57 against 61.
template <int C>
constexpr int gemm_min_s() { return 9; }
template <int C>
constexpr int gemm_min_s_gu() { return C == C_I8 ? 9 : 8; }

template <int C>
constexpr bool gemm_codec() { return C == C_I8 || C == C_I4 || C == C_FP4 || C == C_FP8 || C == C_F16; }

// Code registers per step: GWIN windows x 2 row tiles x Raw, at most 32 VGPRs
// (and as many for the next step's requests), so the formats with more code
// bytes per input take shorter steps: NC >= Raw words.
template <int C>
constexpr int gemm_min_nc() { return (int)(sizeof(typename GemmCodec<C>::Raw) / 4); }

// A grid of fewer blocks than this takes one block per K chunk (split-K).
constexpr size_t GEMM_SPLIT_BELOW = 1024;

// The split-K partials live in one buffer per device that the library keeps
// and grows on demand, up to WS_MAX bytes (larger needs take the unsplit
// kernel).  Every use waits on its stream for the event recorded after the
// previous use, whichever stream that was, so calls on different streams
// take turns with the buffer; a grow first waits on the host for that event.
// A stream under graph capture takes the unsplit kernel, so that no graph
// refers to the buffer.
constexpr size_t WS_MAX = size_t(1) << 30;
struct Workspace {
    std::mutex mu;
    float *buf = nullptr;
    size_t bytes = 0;
    hipEvent_t done = nullptr;   // recorded after the last use
    bool used = false;
};
Workspace g_ws[64];

// Whether k_gemv_mma takes the split-K chunks: one token tile, 4-bit codes
// with one scale per row and 32-input window, whole chunks, 16-byte aligned
// rows of codes and scales.
template <int C, int NC>
bool gemv_mma_fits(const MatDev &m, int S) {
    if constexpr (NC != 1 || (C != C_I4 && C != C_FP4)) {
        return false;
    } else {
        return S <= 16 && m.K % GEMM_KC == 0 && m.shift == 0 && m.srow == 0 && m.sstride % 4 == 0 &&
               m.qstride % 16 == 0 && ((uintptr_t)m.q | (uintptr_t)m.s) % 16 == 0;
    }
}

template <int C, bool GU, int NC>
hipError_t go_gemm_nc(const MatDev &m0, const MatDev &m1, const float *x, int S, float *y, float L,
                      hipStream_t st, const char *name) {
    static_assert(NC >= gemm_min_nc<C>(), "a step's codes must fit 32 registers");
    const int O = m0.O, nch = (m0.K + GEMM_KC - 1) / GEMM_KC;
    const bool gv = gemv_mma_fits<C, NC>(m0, S) && (!GU || gemv_mma_fits<C, NC>(m1, S));
    const int rows_plain = GU ? GROWS / 2 : GROWS;
    const int rows_per_block = gv ? (GU ? 16 : 32) * GV_W : rows_plain;
    dim3 grid((O + rows_plain - 1) / rows_plain, (S + 16 * NC - 1) / (16 * NC));
    const auto plain = [&]() {   // each block walks all of K
        launch(name, (k_gemm<C, GU, NC>), grid, dim3(256), 0, st, m0, m1, x, S, y, L, (float *)nullptr, 0);
        return hipGetLastError();
    };
    if (nch == 1 || (size_t)grid.x * grid.y >= GEMM_SPLIT_BELOW) return plain();
    grid.x = (O + rows_per_block - 1) / rows_per_block;
    const int op = grid.x * rows_per_block;
    const size_t bytes = (size_t)nch * (GU ? 2 : 1) * S * op * sizeof(float);
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(st, &cs);
    if (e != hipSuccess) return e;
    int dev = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if (bytes > WS_MAX || cs != hipStreamCaptureStatusNone || dev < 0 || dev >= 64) return plain();
    Workspace &W = g_ws[dev];
    std::lock_guard<std::mutex> lock(W.mu);
    if (!W.done && (e = hipEventCreateWithFlags(&W.done, hipEventDisableTiming)) != hipSuccess) return e;
    if (W.bytes < bytes) {
        if (W.used && (e = hipEventSynchronize(W.done)) != hipSuccess) return e;
        if (W.buf) (void)hipFree(W.buf);
        W.buf = nullptr;
        W.bytes = 0;
        if ((e = hipMalloc((void **)&W.buf, bytes)) != hipSuccess) return e;
        W.bytes = bytes;
    }
    float *part = W.buf;
    if (W.used && (e = hipStreamWaitEvent(st, W.done, 0)) != hipSuccess) return e;
    if constexpr (NC == 1 && (C == C_I4 || C == C_FP4)) {
        if (gv)
            launch(name, (k_gemv_mma<C, GU>), dim3(grid.x, nch), dim3(WAVE * GV_W), 0, st, m0, m1, x, S, part, op);
    }
    if (!gv) {
        grid.z = nch;
        launch(name, (k_gemm<C, GU, NC>), grid, dim3(256), 0, st, m0, m1, x, S, y, L, part, op);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const size_t n = (size_t)S * O;
    launch("gemm_reduce", (k_gemm_reduce<GU>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, part, nch, S, O,
           op, y, L);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = hipEventRecord(W.done, st)) != hipSuccess) return e;
    W.used = true;
    return hipSuccess;
}

template <int C, bool GU>
hipError_t go_gemm(const MatDev &m0, const MatDev &m1, const float *x, int S, float *y, float L, hipStream_t st) {
    // token tiles per block: fewer for smaller batches, so that the grid has
    // enough blocks (at least 4 token blocks per row block up to 256 tokens)
    const char *name = GU ? "gemm_gate_up" : "gemm";
    // int8 and E4M3 hold twice int4's code registers per step, f16 four times
    if constexpr (gemm_min_nc<C>() <= 1)
        if (S <= 64) return go_gemm_nc<C, GU, 1>(m0, m1, x, S, y, L, st, name);
    if constexpr (gemm_min_nc<C>() <= 2)
        if (S <= 128) return go_gemm_nc<C, GU, 2>(m0, m1, x, S, y, L, st, name);
    return go_gemm_nc<C, GU, 4>(m0, m1, x, S, y, L, st, name);
}

// k_rows_x for 1-4 tokens and K of 1-4 whole 64-chunk steps (int3, whose
// 64-input chunks would spill a wider batch, at one token only, and its
// gate/up pairs at 1-3 steps).
template <int C, bool GU>
bool rows_x_fits(int K, int S) {
    const int unit = WAVE * Codec<C>::CW;
    return S <= (C == C_I3 ? 1 : 4) && K % unit == 0 && K / unit <= (C == C_I3 && GU ? 3 : 4);
}

// Also 1-4 tokens' matmul and gate_up over 6144 inputs in 6 steps of
// 16-input chunks (int8, E4M3 and int8-gs rows) or 12 of 8-input chunks (f16
// and bf16 rows): measured on MI355X, interleaved against the general row
// kernel, 6144^2 matmul at 1 token E4M3 10.39-10.64 -> 8.81-8.84 us, int8-gs
// 10.10-10.27 -> 8.68-8.88, f16 14.89-15.04 -> 12.86-13.17, bf16 14.88 ->
// 12.96-12.99, at 2 and 4 tokens E4M3 12.3-13.2 -> 11.6-11.8 and 17.8-18.2
// -> 15.5-15.6, f16 16.1-16.7 -> 15.9-16.3 and 20.3-20.5 -> 19.7; gate_up on
// two such matrices at 1 token E4M3 17.4-17.6 -> 14.0-14.6, int8-gs
// 16.5-17.1 -> 15.2-15.5, f16 27.8 -> 23.4.  The single expert's launches
// take the same step counts (unit_launch).
template <int C>
bool rows_x_fits_wide1(int K, int S) {
    return S <= 4 && ((Codec<C>::CW == 16 && K == 6 * WAVE * Codec<C>::CW) ||
                      (Codec<C>::CW == 8 && K == 12 * WAVE * Codec<C>::CW));
}

// Bytes of LDS k_rows_x takes: x of SM tokens, and for codes with an
// offset the chunk sums of x.
template <int C, int SM>
size_t rows_x_lds(int K) {
    return ((size_t)SM * x_lds_len<Codec<C>::CW>(K) + (Codec<C>::OFFS != 0.f ? SM * K / Codec<C>::CW : 0)) * 4;
}

template <int C, int SM, bool GU, int NS>
hipError_t go_rows_x(const MatDev &g, const MatDev &u, const float *x, int S, float *y, float L, hipStream_t st,
                     const char *name) {
    const size_t lds = rows_x_lds<C, SM>(g.K);
    if (lds > 160 * 1024) return hipErrorInvalidValue;
    constexpr int W = SM == 1 ? GX_W : GXM_W, R = SM == 1 ? (C == C_I3 ? GX_R : GX1_R) : GXM_R;
    if (g.O >= GX_WIDE_ROWS) {
        launch(name, (k_rows_x<C, SM, GU, NS, W, R>), dim3((g.O + W * R - 1) / (W * R)), dim3(WAVE * W), lds, st,
               g, u, x, S, y, L);
    } else {
        launch(name, (k_rows_x<C, SM, GU, NS, GXS_W, GXS_R>), dim3((g.O + GXS_W * GXS_R - 1) / (GXS_W * GXS_R)),
               dim3(WAVE * GXS_W), lds, st, g, u, x, S, y, L);
    }
    return hipGetLastError();
}

template <int C, bool GU, int SM>
hipError_t rows_x_sm(const MatDev &g, const MatDev &u, const float *x, int S, float *y, float L, hipStream_t st,
                     const char *name) {
    switch (g.K / (WAVE * Codec<C>::CW)) {
    case 1: return go_rows_x<C, SM, GU, 1>(g, u, x, S, y, L, st, name);
    case 2: return go_rows_x<C, SM, GU, 2>(g, u, x, S, y, L, st, name);
    case 3: return go_rows_x<C, SM, GU, 3>(g, u, x, S, y, L, st, name);
    case 6:
        if constexpr (Codec<C>::CW == 16) return go_rows_x<C, SM, GU, 6>(g, u, x, S, y, L, st, name);
        else return hipErrorInvalidValue;   // not taken (rows_x_fits_wide1)
    case 12:
        if constexpr (Codec<C>::CW == 8) return go_rows_x<C, SM, GU, 12>(g, u, x, S, y, L, st, name);
        else return hipErrorInvalidValue;   // not taken (rows_x_fits_wide1)
    default:
        if constexpr (C == C_I3 && GU) return hipErrorInvalidValue;   // not taken (rows_x_fits)
        else return go_rows_x<C, SM, GU, 4>(g, u, x, S, y, L, st, name);
    }
}

template <int C, bool GU>
hipError_t rows_x(const MatDev &g, const MatDev &u, const float *x, int S, float *y, float L, hipStream_t st,
                  const char *name) {
    if (S == 1) return rows_x_sm<C, GU, 1>(g, u, x, S, y, L, st, name);
    if constexpr (C != C_I3) {
        if (S == 2) return rows_x_sm<C, GU, 2>(g, u, x, S, y, L, st, name);
        return rows_x_sm<C, GU, 4>(g, u, x, S, y, L, st, name);
    }
    return hipErrorInvalidValue;
}

template <int C>
hipError_t matmul_c(const MatDev &m, const float *x, int S, float *y, hipStream_t st) {
    if constexpr (gemm_codec<C>())
        if (S >= gemm_min_s<C>() && m.K % 32 == 0) return go_gemm<C, false>(m, m, x, S, y, INFINITY, st);
    if (rows_x_fits<C, false>(m.K, S) || rows_x_fits_wide1<C>(m.K, S))
        return rows_x<C, false>(m, m, x, S, y, INFINITY, st, "matmul");
    // int3's 64-input chunks: 8 tokens at a time would spill, 4 fit with x in LDS
    if constexpr (C != C_I3)
        if (S >= 8) return go_matmul<C, MM_R, 8>(m, x, S, y, st);
    if (S >= 4) return go_matmul<C, MM_R, 4>(m, x, S, y, st);
    if (S >= 2) return go_matmul<C, MM_R, 2>(m, x, S, y, st);
    // one token: int8 and E4M3 rows (16 inputs a chunk) two rows a wave (measured on MI355X, 6144^2
    // interleaved against four: int8-gs 10.6-10.9 -> 10.1-10.4 us, E4M3 10.9-11.0 -> 10.7-10.8; f16 and
    // bf16 lose 3%, one row a wave loses for every format)
    constexpr int R1 = (C == C_I8 || C == C_FP8) ? 2 : MM_R;
    return go_matmul<C, R1, 1>(m, x, S, y, st);
}

template <int C, int R, int SM>
hipError_t go_gate_up(const MatDev &g, const MatDev &u, const float *x, int S, float *h, float L, hipStream_t st) {
    const int rows_per_block = R * WPB;
    dim3 grid((g.O + rows_per_block - 1) / rows_per_block);
    static_assert(SM * WAVE * Codec<C>::CW * 4 <= MM_LDS_BYTES, "64 code chunks of x per token fit the LDS budget");
    const int KC = matmul_kc<C, SM>(g.K);
    launch("gate_up", (k_rows_lds<C, R, SM, true>), grid, dim3(WAVE * WPB),
           (size_t)SM * x_lds_len<Codec<C>::CW>(KC) * 4, st, g, u, x, S, h, KC, L);
    return hipGetLastError();
}

template <int C>
hipError_t gate_up_c(const MatDev &g, const MatDev &u, const float *x, int S, float *h, float L, hipStream_t st) {
    if constexpr (gemm_codec<C>())
        if (S >= gemm_min_s_gu<C>() && g.K % 32 == 0) return go_gemm<C, true>(g, u, x, S, h, L, st);
    if (rows_x_fits<C, true>(g.K, S) || rows_x_fits_wide1<C>(g.K, S)) return rows_x<C, true>(g, u, x, S, h, L, st, "gate_up");
    // int3's 64-input chunks: 8 tokens at a time would spill, 4 fit with x in LDS
    if constexpr (C != C_I3)
        if (S >= 8) return go_gate_up<C, 2, 8>(g, u, x, S, h, L, st);
    if (S >= 4) return go_gate_up<C, 2, 4>(g, u, x, S, h, L, st);
    if (S >= 2) return go_gate_up<C, 4, 2>(g, u, x, S, h, L, st);
    return go_gate_up<C, 4, 1>(g, u, x, S, h, L, st);
}

template <int C>
hipError_t dequant_c(const MatDev &m, float *out, hipStream_t st) {
    const size_t n = (size_t)m.O * (m.K / Codec<C>::CW);
    dim3 grid((unsigned)((n + 255) / 256));
    launch("dequant", (k_dequant<C>), grid, dim3(256), 0, st, m, out);
    return hipGetLastError();
}


// One token, one routed expert, no shared expert, and K (H for gate/up, I
// for down) of k_rows_x's shapes: the unit kernels.
template <int C, bool GU>
bool unit_fits(const GroupArgs &a, int K) {
    return a.S == 1 && a.k == 1 && a.shared < 0 && (rows_x_fits<C, GU>(K, 1) || rows_x_fits_wide1<C>(K, 1)) &&
           rows_x_lds<C, 1>(K) <= 160 * 1024;
}

template <int C, bool GU, int NS, int W, int R>
hipError_t go_unit(const GroupArgs &a, hipStream_t st) {
    const int O = GU ? a.I : a.H, K = GU ? a.H : a.I;
    const dim3 grid((O + W * R - 1) / (W * R)), block(WAVE * W);
    if constexpr (GU)
        launch("group_gate_up", (k_unit_gate_up<C, NS, W, R>), grid, block, rows_x_lds<C, 1>(K), st, a);
    else
        launch("group_down", (k_unit_down<C, NS, W, R>), grid, block, rows_x_lds<C, 1>(K), st, a);
    return hipGetLastError();
}

template <int C, bool GU, int NS>
hipError_t unit_shape(const GroupArgs &a, hipStream_t st) {
    if ((GU ? a.I : a.H) >= GX_WIDE_ROWS) return go_unit<C, GU, NS, GX_W, GX_R>(a, st);
    return go_unit<C, GU, NS, GXS_W, GXS_R>(a, st);
}

template <int C, bool GU>
hipError_t unit_launch(const GroupArgs &a, hipStream_t st) {
    switch ((GU ? a.H : a.I) / (WAVE * Codec<C>::CW)) {
    case 1: return unit_shape<C, GU, 1>(a, st);
    case 2: return unit_shape<C, GU, 2>(a, st);
    case 3: return unit_shape<C, GU, 3>(a, st);
    case 6:
        if constexpr (Codec<C>::CW == 16) return unit_shape<C, GU, 6>(a, st);
        else return hipErrorInvalidValue;   // not taken (unit_fits)
    case 12:
        if constexpr (Codec<C>::CW == 8) return unit_shape<C, GU, 12>(a, st);
        else return hipErrorInvalidValue;   // not taken (unit_fits)
    default:
        if constexpr (C == C_I3 && GU) return hipErrorInvalidValue;   // not taken (unit_fits)
        else return unit_shape<C, GU, 4>(a, st);
    }
}

// Both launches take one slot at a time, at every S: tokens that share an
// expert take further passes over its rows, which the caches then serve.
// (Beyond one token most units serve one slot; 2-slot batches cost the
// gate/up launch its one-token register and LDS budget, 3 waves a SIMD
// against 5: measured on MI355X, int4-g32 group, gate/up 54.2 -> 51.2 us at
// 2 tokens and 108.8 -> 93.6 us at 4 with the shared expert's blocks first.)
template <int C>
hipError_t group_a(const GroupArgs &a, hipStream_t st) {
    if (unit_fits<C, true>(a, a.H)) return unit_launch<C, true>(a, st);
    const int units = a.S * a.k + (a.shared >= 0 ? 1 : 0);
    const int rows_per_block = RA * WPB_A;
    // the slot's row of x, and the chunk sums of x after it
    const size_t lds = ((size_t)x_lds_len<Codec<C>::CW, GROUP_XPAD>(a.H) + (size_t)a.H / Codec<C>::CW) * sizeof(float);
    dim3 grid((a.I + rows_per_block - 1) / rows_per_block, units);
    if constexpr (C != C_I3)
        launch("group_gate_up", (k_group_gate_up1<C, RA>), grid, dim3(WAVE * WPB_A), lds, st, a);
    else
        launch("group_gate_up", (k_group_gate_up<C, RA>), grid, dim3(WAVE * WPB_A), lds, st, a);
    return hipGetLastError();
}

template <int C>
hipError_t group_b(const GroupArgs &a, hipStream_t st) {
    if (unit_fits<C, false>(a, a.I)) return unit_launch<C, false>(a, st);
    const int units = a.S * a.k + (a.shared >= 0 ? a.S : 0);   // each shared slot a unit
    const int slots = a.S * a.k + (a.shared >= 0 ? a.S : 0);
    const size_t v4_lds = a.act == ACT_SWIGLU_V4 ? 2 * (size_t)a.S * a.k * sizeof(int) : 0;
    if constexpr (C != C_I3) {
        if (a.S == 1 && a.shared >= 0 && a.k >= 6 && a.k <= 8 && a.I == WAVE * Codec<C>::CW &&
            (long)(a.k + 1) * a.I / 4 <= (long)SPLIT_HN * WAVE * 2 * a.k) {
            dim3 grid((a.H + SPLIT_R - 1) / SPLIT_R);
            const size_t lds = ((size_t)(a.k + 1) * a.I + (size_t)slots * SPLIT_R) * sizeof(float) + v4_lds;
            launch("group_down", (k_group_down_split<C>), grid, dim3(WAVE * 2 * a.k), lds, st, a);
            return hipGetLastError();
        }
    }
    const int waves = units < DOWN_MAX_WAVES ? units : DOWN_MAX_WAVES;
    if (a.H > DOWN_ROUND * RB && a.H <= DOWN_ROUND * RB_WIDE) {
        dim3 grid((a.H + RB_WIDE - 1) / RB_WIDE);
        const size_t lds = (size_t)slots * RB_WIDE * sizeof(float) + v4_lds;
        launch("group_down", (k_group_down<C, RB_WIDE>), grid, dim3(WAVE * waves), lds, st, a);
        return hipGetLastError();
    }
    dim3 grid((a.H + RB - 1) / RB);
    // the slots' outputs; DeepSeek V4's combine adds the ids and their order
    const size_t lds = (size_t)slots * RB * sizeof(float) + v4_lds;
    launch("group_down", (k_group_down<C, RB>), grid, dim3(WAVE * waves), lds, st, a);
    return hipGetLastError();
}

// Calls f(std::integral_constant<int, C>) for the codec of a run-time id.
template <typename F>
hipError_t with_codec(int codec, F &&f) {
    switch (codec) {
    case C_I8: return f(std::integral_constant<int, C_I8>{});
    case C_I4: return f(std::integral_constant<int, C_I4>{});
    case C_I3: return f(std::integral_constant<int, C_I3>{});
    case C_FP4: return f(std::integral_constant<int, C_FP4>{});
    case C_F32: return f(std::integral_constant<int, C_F32>{});
    case C_BF16: return f(std::integral_constant<int, C_BF16>{});
    case C_FP8: return f(std::integral_constant<int, C_FP8>{});
    case C_F16: return f(std::integral_constant<int, C_F16>{});
    }
    return hipErrorInvalidValue;
}

// The library-held expert-group scratch of dqg_expert_group_noalloc, one
// copy per device for the life of the process.  In host code `scratch` is
// only a stand-in for the symbol: its device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) uint8_t scratch[STATIC_SCRATCH_BYTES];

struct StaticScratch {
    std::once_flag once;
    hipError_t err = hipSuccess;
    void *ptr = nullptr;
};
StaticScratch g_static[64];

}  // namespace

hipError_t static_scratch(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    StaticScratch &s = g_static[dev];
    std::call_once(s.once, [&] { s.err = hipGetSymbolAddress(&s.ptr, HIP_SYMBOL(scratch)); });
    if (s.err != hipSuccess) return s.err;
    *ptr = s.ptr;
    return hipSuccess;
}

hipError_t launch_matmul(int codec, const MatDev &m, const float *x, int S, float *y, hipStream_t st) {
    return with_codec(codec, [&](auto c) { return matmul_c<decltype(c)::value>(m, x, S, y, st); });
}

hipError_t launch_gate_up(int codec, const MatDev &g, const MatDev &u, const float *x, int S,
                          float *h, float limit, hipStream_t st) {
    return with_codec(codec, [&](auto c) { return gate_up_c<decltype(c)::value>(g, u, x, S, h, limit, st); });
}

hipError_t launch_route(const RouteArgs &a, hipStream_t st) {
    const dim3 grid((a.S + ROUTE_WAVES - 1) / ROUTE_WAVES), block(WAVE * ROUTE_WAVES);
    if (a.E <= 64) launch("route", k_route<1>, grid, block, 0, st, a);
    else if (a.E <= 128) launch("route", k_route<2>, grid, block, 0, st, a);
    else if (a.E <= 256) launch("route", k_route<4>, grid, block, 0, st, a);
    else if (a.E <= 512) launch("route", k_route<8>, grid, block, 0, st, a);
    else if (a.E <= ROUTE_MAX_E) launch("route", k_route<16>, grid, block, 0, st, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_read(const void *p, uint64_t nbytes, uint32_t *sink, int cus, hipStream_t st) {
    launch("read", k_read, dim3(8 * cus), dim3(256), 0, st, (const u32x4 *)p, nbytes / 1024, sink);
    return hipGetLastError();
}

hipError_t launch_dequant(int codec, const MatDev &m, float *out, hipStream_t st) {
    return with_codec(codec, [&](auto c) { return dequant_c<decltype(c)::value>(m, out, st); });
}

hipError_t launch_group(int codec_gu, int codec_down, const GroupArgs &a, hipStream_t st, int *launches) {
    hipError_t e = with_codec(codec_gu, [&](auto c) { return group_a<decltype(c)::value>(a, st); });
    if (e != hipSuccess) return e;
    ++*launches;
    if (a.act == ACT_SWIGLU_V4) {
        const int slots = a.S * a.k + (a.shared >= 0 ? a.S : 0);
        const int nblk = slots * (a.I / 128);
        launch("group_act_v4", k_group_act_v4, dim3((nblk + 3) / 4), dim3(256), 0, st, a.h, nblk);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        ++*launches;
    }
    e = with_codec(codec_down, [&](auto c) { return group_b<decltype(c)::value>(a, st); });
    if (e == hipSuccess) ++*launches;
    return e;
}

}  // namespace dqg
