// Shared device helpers of the gfx950 kernels (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mmdit.h"

#define MMDIT_DEV __device__ __forceinline__

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));   // 32 fp8 codes

namespace mmdit {

// bf16 bits -> fp32 (exact)
MMDIT_DEV float bf2f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16 bits, round to nearest even (the conversion instruction of gfx950)
MMDIT_DEV uint16_t f2bf(float f) {
    __bf16 h = static_cast<__bf16>(f);
    return __builtin_bit_cast(uint16_t, h);
}

// two fp32 -> packed bf16 pair (low = a)
MMDIT_DEV uint32_t pack2bf(float a, float b) {
    return uint32_t(f2bf(a)) | (uint32_t(f2bf(b)) << 16);
}

// fp32 -> fp16 bits, round to nearest even
MMDIT_DEV uint16_t f2h(float f) {
    _Float16 h = static_cast<_Float16>(f);
    return __builtin_bit_cast(uint16_t, h);
}

// two fp32 -> packed fp16 pair (low = a)
MMDIT_DEV uint32_t pack2h(float a, float b) {
    return uint32_t(f2h(a)) | (uint32_t(f2h(b)) << 16);
}

// fp16 bits -> fp32 (exact)
MMDIT_DEV float h2f(uint16_t b) { return static_cast<float>(__builtin_bit_cast(_Float16, b)); }

// Sum over all 64 lanes of a wavefront; every lane gets the total. Lane
// exchanges without LDS round trips: DPP within each row of 16 lanes (swap
// neighbours, swap pairs, mirror each half row, mirror the row: after each
// step every lane holds the sum of a twice larger aligned group), then the
// row swaps of gfx950 (permlane16 / permlane32) across rows. A fixed
// sequence, so the result does not depend on timing.
// Smallest e with 2^e >= b for b >= 0 (0 for b = 0): frexp is exact.
MMDIT_DEV int ceil_log2_exp(float b) {
    int e = 0;
    const float m = frexpf(b, &e);
    return m == 0.5f ? e - 1 : (m == 0.0f ? 0 : e);
}

MMDIT_DEV float wave_sum(float v) {
    v += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0xB1, 0xF, 0xF, false));  // lane ^ 1
    v += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0x4E, 0xF, 0xF, false));  // lane ^ 2
    v += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0x141, 0xF, 0xF, false)); // half-row mirror
    v += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0x140, 0xF, 0xF, false)); // row mirror
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);   // rows 0+1, 2+3
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

// Sum over aligned groups of G lanes (G a power of two <= 64).
template <int G>
MMDIT_DEV float group_sum(float v) {
#pragma unroll
    for (int o = G / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// SiLU(x) = x / (1 + e^-x)
// The reciprocals below use the hardware's v_rcp_f32 (within 1 ulp) instead
// of a correctly rounded division: a GEMM epilogue evaluates one per output
// element, and the division's fix-up sequence costs ~8 more VALU operations
// that delay the matrix cores of the same SIMD. rcp(inf) = 0 keeps both
// functions exact in their saturated ranges.
MMDIT_DEV float silu(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// GELU, tanh form: 0.5 x (1 + tanh(u)), u = sqrt(2/pi) (x + 0.044715 x^3).
// 0.5 (1 + tanh u) = 1 / (1 + e^{-2u}), and e^{-2u} = 2^{x (c1 + c2 x^2)} with
// c1 = -2 log2(e) sqrt(2/pi), c2 = 0.044715 c1: one exp2, one reciprocal and
// five multiplies and adds per value (the epilogue of the MLP-in projection runs
// this while the compute unit's matrix cores wait). Saturates to 0 and x.
MMDIT_DEV float gelu_tanh(float x) {
    const float c1 = -2.302208198144325f;
    const float c2 = -0.1029432395800235f;
    const float e = __builtin_amdgcn_exp2f(x * fmaf(c2, x * x, c1));
    return x * __builtin_amdgcn_rcpf(1.0f + e);
}

}  // namespace mmdit

// Launchers (defined in the kernel sources, called by the API layer). Each
// returns hipSuccess or the launch error.
namespace mmdit {

hipError_t launch_ln_modulate(const float* x, int rows, int hidden, int split,
                              const float* shift0, const float* scale0,
                              const float* shift1, const float* scale1, float eps,
                              uint16_t* out, hipStream_t s,
                              uint8_t* codes = nullptr, float* qscale = nullptr);

hipError_t launch_qknorm_rope(const uint16_t* qkv, int ld, int seq_len, int heads, int head_dim,
                              int split, const uint16_t* qn0, const uint16_t* kn0,
                              const uint16_t* qn1, const uint16_t* kn1, const float* rope,
                              float eps, int l_pad, uint16_t* q_out, uint16_t* k_out,
                              uint16_t* vt_out, hipStream_t s);

hipError_t launch_attention(const uint16_t* q, const uint16_t* k, const uint16_t* vt, int heads,
                            int seq_len, int head_dim, int l_pad, uint16_t* out, int ldo,
                            hipStream_t s);

// One GEMM group: rows [row0, row0 + m) of A / out share one weight set.
struct GemmGroup {
    int row0, m;
    const void* w;
    const float* scale;
    const uint16_t* bias;
    const float* gate;
    const uint16_t* qn;   // EPI_QKV_ATTN: RMSNorm scales [D] of q and k (bf16)
    const uint16_t* kn;
};

// Internal epilogue of the double block's QKV projection (not accepted by the
// per-kernel entry): columns [q | k | v] of the joint sequence; q and k get
// per-head RMSNorm and RoPE and go to [heads, l_pad, D], v to the transposed,
// quad-swapped [heads, D, l_pad] layout the attention kernel reads.
// Internal weight type (not in the ABI's enum): OCP e4m3 weight codes with an
// fp32 scale per output channel, against 16-bit (fp16) activations; each
// weight fragment is decoded to fp16 in registers (exact) and the scale
// multiplies the fp32 sum, as for int8 codes. The fp8 denoise step uses it
// for its patch embedding, final projection and batched modulation, whose
// activation operands stay 16-bit.
constexpr int WT_FP8_W16A = 16;

constexpr int EPI_QKV_ATTN = 64;
// The single-stream block's linear1 ([q | k | v | mlp] columns): the split
// GELU / SwiGLU epilogues whose first split_n = 3H columns take the
// EPI_QKV_ATTN path (a separate kernel per variant keeps registers in bounds).
constexpr int EPI_SPLIT_GELU_ATTN = 65;
constexpr int EPI_SPLIT_SWIGLU_ATTN = 66;
// The public epilogue an internal one behaves as outside the q|k|v columns.
constexpr int epi_base(int e) {
    return e == EPI_SPLIT_GELU_ATTN ? MMDIT_EPI_SPLIT_GELU : e == EPI_SPLIT_SWIGLU_ATTN ? MMDIT_EPI_SPLIT_SWIGLU : e;
}

struct GemmArgs {
    int n, k;
    int wtype;   // enum mmdit_weight_dtype
    const uint16_t* a;
    int lda;
    int epilogue;
    void* out;
    int ldo;
    const float* resid;
    int ldr;
    int split_n;
    void* out2;
    int ldo2;
    int out2_col;
    float alpha;
    int ngroups;
    GemmGroup g[2];
    // Set by the launcher: the last tail_rows row tiles (of both groups'
    // row tiles stacked) run as 128-wide tiles after the full_tiles 256-wide
    // ones, so that a partial last round of 256-wide tiles becomes half as long.
    int tail_rows;
    int full_tiles;
    // Set by the launcher: the first head_rows row tiles run as 128-wide
    // tiles ahead of the 256-wide ones (0: none).
    int head_rows;
    const float* a_scale;   // fp32 per row of A, fp8 operands only
    // EPI_QKV_ATTN only
    uint16_t* q_out;        // [heads, l_pad, D] bf16
    uint16_t* k_out;
    uint16_t* vt_out;       // [heads, D, l_pad] bf16
    int l_pad, head_dim;
    const float* rope;      // [L, D/2, 2] fp32 (cos, sin) per pair
    float rms_eps;
    // fp8 operands only: q and k written as e4m3 codes ([heads, l_pad, D]
    // bytes, q_out / k_out unused) at the power-of-two scales 2^eq, 2^ek
    // that the q / k norm scales bound (the fp8 attention's operands)
    uint8_t* q8_out;
    uint8_t* k8_out;
    const uint16_t* fp8_norms[4];   // q text, q image, k text, k image ([D] bf16)
    float fp8_bound;                // fl32(sqrt(D) / 448)
    int* fp8_exps;                  // (eq, ek), written by the first column tiles
};

// Rows [seq_len, l_pad) of the attention operands as zeros.
hipError_t launch_zero_attn_pad(uint16_t* q, uint16_t* k, uint16_t* vt, int heads, int head_dim, int seq_len,
                                int l_pad, hipStream_t s);

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s);

struct GemvSet {
    const void* w;          // [n, k] bf16 / fp16 / int8 codes
    const float* scale;     // [n], int8 only
    const uint16_t* bias;   // [n] bf16
    float* out;             // [n] fp32
};
struct GemvSets {
    int count;              // 1 or 2
    GemvSet s[2];
};

// k <= 4096 and a multiple of 16
hipError_t launch_gemv(const float* x, int k, int n, int wtype, int silu_input, int accumulate,
                       const GemvSets& sets, hipStream_t s);

// bf16 -> fp16 (round to nearest even), count elements
hipError_t launch_bf16_to_f16(const uint16_t* src, uint16_t* dst, size_t count, hipStream_t s);

// out[0:256] = emb(t), out[256:512] = emb(g)
hipError_t launch_time_and_guidance_embedding(float t, float g, float* out, hipStream_t s);

hipError_t launch_euler(float* z, const float* v, int64_t n, float dt, hipStream_t s);

hipError_t launch_rope_table(const int32_t* ids, int seq_len, int head_dim, int a0, int a1, int a2,
                             float theta, float* rope, hipStream_t s);

hipError_t launch_copy_f32(float* dst, const float* src, int64_t n, hipStream_t s);

// Per-row fp8 e4m3 quantisation of 16-bit rows (bf16 when x_bf16, else fp16)
hipError_t launch_quantize_fp8_rows(const uint16_t* x, bool x_bf16, int rows, int cols, int ldx,
                                    uint8_t* codes, int ldc, float* scales, hipStream_t s);

// y fp16 = SiLU(x fp32), n elements
// fp8 attention (k_attention_fp8.hip): q, k, v^T to e4m3 (exps[0..1] = eq, ek),
// then the attention on the codes
hipError_t launch_quantize_vt_fp8(const uint16_t* vt, int heads, int head_dim, int l_pad, uint8_t* vt8, float* sv,
                                  hipStream_t s);
hipError_t launch_quantize_attention_fp8(const uint16_t* q, const uint16_t* k, const uint16_t* vt, int heads,
                                         int head_dim, int l_pad, const uint16_t* gq0, const uint16_t* gq1,
                                         const uint16_t* gk0, const uint16_t* gk1, uint8_t* q8, uint8_t* k8,
                                         uint8_t* vt8, float* sv, int* exps, hipStream_t s);
hipError_t launch_attention_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* vt8, const float* sv,
                                const int* exps, int heads, int seq_len, int head_dim, int l_pad, uint16_t* out,
                                int ldo, hipStream_t s);
hipError_t launch_silu_to_f16(const float* x, uint16_t* y, int64_t n, hipStream_t s);

}  // namespace mmdit
