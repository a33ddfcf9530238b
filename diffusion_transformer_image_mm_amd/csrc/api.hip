// C ABI of libmmdit.so: argument validation, workspace carving and the
// orchestration of the block / step kernels on one stream.
#include <atomic>
#include <cmath>

#include "common.h"

using namespace mmdit;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v, size_t a = kAlign) { return (v + a - 1) / a * a; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dtype_ok(int dt) { return dt == MMDIT_BF16 || dt == MMDIT_INT8 || dt == MMDIT_F16 || dt == MMDIT_FP8; }

// Validate the sizes of a model. Returns MMDIT_OK or the status.
int check_dims(const mmdit_dims* d) {
    if (!d) return MMDIT_E_NULL;
    if (d->head_dim != 64 && d->head_dim != 128) return MMDIT_E_SHAPE;
    if (d->heads < 1 || d->hidden != d->heads * d->head_dim) return MMDIT_E_SHAPE;
    if (d->hidden % 64 != 0 || d->hidden > 4096) return MMDIT_E_SHAPE;
    if (d->mlp_hidden < 64 || d->mlp_hidden % 64 != 0 || d->mlp_hidden > 65536) return MMDIT_E_SHAPE;
    if (d->txt_len < 1 || d->img_len < 1) return MMDIT_E_SHAPE;
    if ((int64_t)d->txt_len + d->img_len > (1 << 20)) return MMDIT_E_SHAPE;
    int sum = 0;
    for (int a = 0; a < 3; ++a) {
        if (d->rope_axes[a] < 0 || d->rope_axes[a] % 2 != 0) return MMDIT_E_SHAPE;
        sum += d->rope_axes[a];
    }
    if (sum != d->head_dim) return MMDIT_E_SHAPE;
    if (!(d->ln_eps > 0.f) || !(d->rms_eps > 0.f) || !(d->rope_theta > 1.f)) return MMDIT_E_SHAPE;
    if (!dtype_ok(d->weight_dtype)) return MMDIT_E_DTYPE;
    if (d->mlp_act != MMDIT_ACT_GELU_TANH && d->mlp_act != MMDIT_ACT_SWIGLU) return MMDIT_E_ARG;
    // fp8 blocks: GELU MLPs only (the SwiGLU epilogues take 16-bit operands)
    if (d->weight_dtype == MMDIT_FP8 && d->mlp_act != MMDIT_ACT_GELU_TANH) return MMDIT_E_DTYPE;
    // fp8 GEMMs take 128 k per stage: every projection's k (H, M, H + M)
    if (d->weight_dtype == MMDIT_FP8 && (d->hidden % 128 != 0 || d->mlp_hidden % 128 != 0))
        return MMDIT_E_SHAPE;
    // SwiGLU GEMM tiles hold 128 features and never straddle the q|k|v / MLP
    // split of the single-stream linear1 (at 3H)
    if (d->mlp_act == MMDIT_ACT_SWIGLU && (d->hidden % 256 != 0 || d->mlp_hidden % 128 != 0))
        return MMDIT_E_SHAPE;
    if (d->guidance_embed != 0 && d->guidance_embed != 1) return MMDIT_E_ARG;
    if (d->ref_len < 0 || d->ref_len >= d->img_len) return MMDIT_E_SHAPE;
    return MMDIT_OK;
}

// fc1 / MLP-part output columns of linear1: M (GELU) or [gate | up] = 2M (SwiGLU)
int mlp_cols(const mmdit_dims* d) {
    return d->mlp_act == MMDIT_ACT_SWIGLU ? 2 * d->mlp_hidden : d->mlp_hidden;
}

int check_ptr(const void* p) {
    if (!p) return MMDIT_E_NULL;
    if (!aligned16(p)) return MMDIT_E_ALIGN;
    return MMDIT_OK;
}

int check_linear(const mmdit_linear& l, int dtype) {
    int st;
    if ((st = check_ptr(l.w)) != MMDIT_OK) return st;
    if ((st = check_ptr(l.bias)) != MMDIT_OK) return st;
    if (dtype == MMDIT_INT8 || dtype == MMDIT_FP8) {
        if (!l.scale) return MMDIT_E_DTYPE;
        if (!aligned16(l.scale)) return MMDIT_E_ALIGN;
    }
    return MMDIT_OK;
}

#define MMDIT_TRY(expr)               \
    do {                              \
        int _st = (expr);             \
        if (_st != MMDIT_OK) return _st; \
    } while (0)

#define MMDIT_HIP(expr)                          \
    do {                                         \
        if ((expr) != hipSuccess) return MMDIT_E_HIP; \
    } while (0)

int stream_weights_ok(const mmdit_stream_weights& s, int dt) {
    MMDIT_TRY(check_linear(s.mod, dt));
    MMDIT_TRY(check_linear(s.qkv, dt));
    MMDIT_TRY(check_linear(s.proj, dt));
    MMDIT_TRY(check_linear(s.fc1, dt));
    MMDIT_TRY(check_linear(s.fc2, dt));
    MMDIT_TRY(check_ptr(s.q_norm));
    MMDIT_TRY(check_ptr(s.k_norm));
    return MMDIT_OK;
}

int double_weights_ok(const mmdit_double_weights* w, int dt) {
    if (!w) return MMDIT_E_NULL;
    MMDIT_TRY(stream_weights_ok(w->txt, dt));
    MMDIT_TRY(stream_weights_ok(w->img, dt));
    return MMDIT_OK;
}

int single_weights_ok(const mmdit_single_weights* w, int dt) {
    if (!w) return MMDIT_E_NULL;
    MMDIT_TRY(check_linear(w->mod, dt));
    MMDIT_TRY(check_linear(w->linear1, dt));
    MMDIT_TRY(check_linear(w->linear2, dt));
    MMDIT_TRY(check_ptr(w->q_norm));
    MMDIT_TRY(check_ptr(w->k_norm));
    return MMDIT_OK;
}

// ---------------------------------------------------------------- workspace
int seq_len(const mmdit_dims* d) { return d->txt_len + d->img_len; }
int padded_len(const mmdit_dims* d) { return (seq_len(d) + 127) / 128 * 128; }

struct Carver {
    char* base;
    size_t off = 0;
    explicit Carver(void* b) : base(static_cast<char*>(b)) {}
    template <class T>
    T* take(size_t count) {
        T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
        off = align_up(off + count * sizeof(T));
        return p;
    }
};

struct DoubleWs {
    float* mod;      // [2][6H] fp32
    uint16_t* h;     // [L, H] fp16 (LayerNorm + modulate output)
    uint16_t* qkv;   // [L, 3H] bf16
    uint16_t* q;     // [heads, l_pad, D] bf16
    uint16_t* k;
    uint16_t* vt;    // [heads, D, l_pad] bf16
    uint16_t* o;     // [L, H] fp16 (attention output)
    uint16_t* a;     // [L, M] fp16 (GELU hidden)
    // fp8 blocks only: the projections' operands as e4m3 codes + row scales
    uint8_t* h8;     // [L, H]
    uint8_t* o8;     // [L, H]
    uint8_t* a8;     // [L, M]
    float* sh;       // [L]
    float* so;       // [L]
    float* sa;       // [L]
    // fp8 attention operands: q, k, v^T codes, per-channel v scales, exponents
    uint8_t* q8;     // [heads, l_pad, D]
    uint8_t* k8;
    uint8_t* vt8;    // [heads, D, l_pad]
    float* sv;       // [H]
    int* exps;       // [2]
};

DoubleWs carve_double(const mmdit_dims* d, Carver& c) {
    const size_t L = seq_len(d), H = d->hidden, M = d->mlp_hidden, LP = padded_len(d);
    DoubleWs w;
    w.mod = c.take<float>(12 * H);
    w.h = c.take<uint16_t>(L * H);
    w.qkv = c.take<uint16_t>(L * 3 * H);
    w.q = c.take<uint16_t>(LP * H);
    w.k = c.take<uint16_t>(LP * H);
    w.vt = c.take<uint16_t>(LP * H);
    w.o = c.take<uint16_t>(L * H);
    w.a = c.take<uint16_t>(L * M);
    w.h8 = w.o8 = w.a8 = nullptr;
    w.sh = w.so = w.sa = nullptr;
    if (d->weight_dtype == MMDIT_FP8) {
        w.h8 = c.take<uint8_t>(L * H);
        w.o8 = c.take<uint8_t>(L * H);
        w.a8 = c.take<uint8_t>(L * M);
        w.sh = c.take<float>(L);
        w.so = c.take<float>(L);
        w.sa = c.take<float>(L);
        w.q8 = c.take<uint8_t>(LP * H);
        w.k8 = c.take<uint8_t>(LP * H);
        w.vt8 = c.take<uint8_t>(LP * H);
        w.sv = c.take<float>(H);
        w.exps = c.take<int>(2);
    } else {
        w.q8 = w.k8 = w.vt8 = nullptr;
        w.sv = nullptr;
        w.exps = nullptr;
    }
    return w;
}

struct SingleWs {
    float* mod;      // [3H] fp32
    uint16_t* h;     // [L, H] fp16
    uint16_t* qkv;   // [L, 3H] bf16
    uint16_t* q;
    uint16_t* k;
    uint16_t* vt;
    uint16_t* cat;   // [L, H + M] fp16: [attention | GELU(mlp)]
    uint8_t* h8;     // fp8 blocks only: [L, H] and [L, H + M] e4m3 codes + row scales
    uint8_t* cat8;
    float* sh;
    float* sc;
    uint8_t* q8;     // fp8 attention operands, as in the double block
    uint8_t* k8;
    uint8_t* vt8;
    float* sv;
    int* exps;
};

SingleWs carve_single(const mmdit_dims* d, Carver& c) {
    const size_t L = seq_len(d), H = d->hidden, M = d->mlp_hidden, LP = padded_len(d);
    SingleWs w;
    w.mod = c.take<float>(3 * H);
    w.h = c.take<uint16_t>(L * H);
    w.qkv = c.take<uint16_t>(L * 3 * H);
    w.q = c.take<uint16_t>(LP * H);
    w.k = c.take<uint16_t>(LP * H);
    w.vt = c.take<uint16_t>(LP * H);
    w.cat = c.take<uint16_t>(L * (H + M));
    w.h8 = w.cat8 = nullptr;
    w.sh = w.sc = nullptr;
    if (d->weight_dtype == MMDIT_FP8) {
        w.h8 = c.take<uint8_t>(L * H);
        w.cat8 = c.take<uint8_t>(L * (H + M));
        w.sh = c.take<float>(L);
        w.sc = c.take<float>(L);
        w.q8 = c.take<uint8_t>(LP * H);
        w.k8 = c.take<uint8_t>(LP * H);
        w.vt8 = c.take<uint8_t>(LP * H);
        w.sv = c.take<float>(H);
        w.exps = c.take<int>(2);
    } else {
        w.q8 = w.k8 = w.vt8 = nullptr;
        w.sv = nullptr;
        w.exps = nullptr;
    }
    return w;
}

struct StepWs {
    float* emb;      // [512]
    float* tmp;      // [2H]
    float* vec;      // [H]
    float* fmod;     // [2H]
    float* x;        // [L, H]
    uint16_t* z16;   // [L_i, C] fp16
    char* blocks;    // shared by the block calls
    size_t block_bytes;
};

size_t block_ws_bytes(const mmdit_dims* d) {
    Carver c1(nullptr), c2(nullptr);
    carve_double(d, c1);
    carve_single(d, c2);
    return c1.off > c2.off ? c1.off : c2.off;
}

StepWs carve_step(const mmdit_dims* d, Carver& c) {
    const size_t L = seq_len(d), H = d->hidden;
    StepWs w;
    w.emb = c.take<float>(512);
    w.tmp = c.take<float>(2 * H);
    w.vec = c.take<float>(H);
    w.fmod = c.take<float>(2 * H);
    w.x = c.take<float>(L * H);
    w.z16 = c.take<uint16_t>((size_t)d->img_len * d->in_channels);
    w.block_bytes = block_ws_bytes(d);
    w.blocks = c.take<char>(w.block_bytes);
    return w;
}

// ---------------------------------------------------------------- helpers
GemvSet gemv_set(const mmdit_linear& l, float* out) {
    GemvSet g;
    g.w = l.w;
    g.scale = l.scale;
    g.bias = l.bias;
    g.out = out;
    return g;
}

hipError_t gemv(const float* x, int k, const mmdit_linear& l, int n, int dt, int silu_in, int acc,
                float* out, hipStream_t s) {
    GemvSets g = {};
    g.count = 1;
    g.s[0] = gemv_set(l, out);
    return launch_gemv(x, k, n, dt, silu_in, acc, g, s);
}

// two weight sets of the same shape over the same input, one launch
hipError_t gemv_2(const float* x, int k, const mmdit_linear& l0, float* out0, const mmdit_linear& l1,
                  float* out1, int n, int dt, int silu_in, hipStream_t s) {
    GemvSets g = {};
    g.count = 2;
    g.s[0] = gemv_set(l0, out0);
    g.s[1] = gemv_set(l1, out1);
    return launch_gemv(x, k, n, dt, silu_in, 0, g, s);
}

GemmGroup group(int row0, int m, const mmdit_linear& l, const float* gate = nullptr) {
    GemmGroup g = {};
    g.row0 = row0;
    g.m = m;
    g.w = l.w;
    g.scale = l.scale;
    g.bias = l.bias;
    g.gate = gate;
    return g;
}

GemmArgs gemm_base(int n, int k, int dt, const uint16_t* a, int lda, int epi, void* out, int ldo) {
    GemmArgs g = {};
    g.n = n;
    g.k = k;
    g.wtype = dt;
    g.a = a;
    g.lda = lda;
    g.epilogue = epi;
    g.out = out;
    g.ldo = ldo;
    return g;
}

hipError_t gemm_2(GemmArgs g, const GemmGroup& g0, const GemmGroup& g1, hipStream_t s) {
    g.ngroups = 2;
    g.g[0] = g0;
    g.g[1] = g1;
    return launch_gemm(g, s);
}

hipError_t gemm_1(GemmArgs g, const GemmGroup& g0, hipStream_t s) {
    g.ngroups = 1;
    g.g[0] = g0;
    return launch_gemm(g, s);
}

// fp8 blocks: the 16-bit activation rows x [rows, cols] as e4m3 codes + row scales
hipError_t quant_rows(const uint16_t* x, int rows, int cols, uint8_t* q, float* sc, hipStream_t s) {
    return launch_quantize_fp8_rows(x, false, rows, cols, cols, q, cols, sc, s);
}

// The projection's activation operand: the fp16 rows themselves, or their fp8
// codes (quantised here) with a row scale for fp8 weights.
GemmArgs proj_base(const mmdit_dims* d, int n, int k, const uint16_t* a16, uint8_t* a8, float* sa, int epi,
                   void* out, int ldo) {
    if (d->weight_dtype != MMDIT_FP8) return gemm_base(n, k, d->weight_dtype, a16, k, epi, out, ldo);
    GemmArgs g = gemm_base(n, k, MMDIT_FP8, reinterpret_cast<const uint16_t*>(a8), k, epi, out, ldo);
    g.a_scale = sa;
    return g;
}

// fp32 latent -> fp16 activation operand of the patch-embedding projection
__global__ void f32_to_f16_kernel(const float* __restrict__ x, uint16_t* __restrict__ y, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        y[i] = f2h(x[i]);
}

// fp8 blocks: the attention-layout epilogue writes q and k as e4m3 codes at
// the power-of-two scales bounded by these norm scales (the fp8 attention's
// operand quantiser, fused) and stores the exponents
void set_fp8_qk(GemmArgs& g, const mmdit_dims* d, uint8_t* q8, uint8_t* k8, int* exps, const uint16_t* qn0,
                const uint16_t* qn1, const uint16_t* kn0, const uint16_t* kn1) {
    g.q8_out = q8;
    g.k8_out = k8;
    g.fp8_norms[0] = qn0;
    g.fp8_norms[1] = qn1;
    g.fp8_norms[2] = kn0;
    g.fp8_norms[3] = kn1;
    g.fp8_bound = (float)(sqrt((double)d->head_dim) / 448.0);
    g.fp8_exps = exps;
}

// ---------------------------------------------------------------- blocks
// premod: the block's modulation [txt 6H | img 6H] computed beforehand
// (mmdit_modulation_batch), or null to compute it here from vec
int run_double(const mmdit_dims* d, const mmdit_double_weights* w, const float* vec, const float* rope,
               const float* x_in, float* x_out, const DoubleWs& ws, hipStream_t s,
               const float* premod = nullptr) {
    const int Lt = d->txt_len, Li = d->img_len, L = Lt + Li, H = d->hidden, M = d->mlp_hidden;
    const int dt = d->weight_dtype, LP = padded_len(d);
    const float* mt = premod ? premod : ws.mod;
    const float* mi = mt + 6 * H;
    // a1: modulation of each stream
    if (!premod) MMDIT_HIP(gemv_2(vec, H, w->txt.mod, ws.mod, w->img.mod, ws.mod + 6 * H, 6 * H, dt, 1, s));
    const bool fp8 = dt == MMDIT_FP8;
    // a2: LN1 + modulate
    // (fp8 blocks: the LayerNorm kernel writes the e4m3 codes and row scales itself)
    MMDIT_HIP(launch_ln_modulate(x_in, L, H, Lt, mt, mt + H, mi, mi + H, d->ln_eps, ws.h, s,
                                 fp8 ? ws.h8 : nullptr, fp8 ? ws.sh : nullptr));
    if (H % 256 == 0) {
        // a3 + a4: QKV projection whose epilogue applies the per-head
        // RMSNorm of q and k and RoPE and writes q, k and v^T in the layout
        // the attention kernel reads (a 256-wide tile lies in one of q|k|v)
        GemmArgs g = proj_base(d, 3 * H, H, ws.h, ws.h8, ws.sh, EPI_QKV_ATTN, nullptr, 0);
        g.split_n = 3 * H;
        g.q_out = ws.q;
        g.k_out = ws.k;
        g.vt_out = ws.vt;
        g.l_pad = LP;
        g.head_dim = d->head_dim;
        g.rope = rope;
        g.rms_eps = d->rms_eps;
        GemmGroup gt = group(0, Lt, w->txt.qkv), gi = group(Lt, Li, w->img.qkv);
        gt.qn = w->txt.q_norm;
        gt.kn = w->txt.k_norm;
        gi.qn = w->img.q_norm ? w->img.q_norm : w->txt.q_norm;
        gi.kn = w->img.k_norm ? w->img.k_norm : w->txt.k_norm;
        if (fp8) set_fp8_qk(g, d, ws.q8, ws.k8, ws.exps, gt.qn, gi.qn, gt.kn, gi.kn);
        MMDIT_HIP(gemm_2(g, gt, gi, s));
        MMDIT_HIP(launch_zero_attn_pad(ws.q, ws.k, ws.vt, d->heads, d->head_dim, L, LP, s));
    } else {
        // a3: QKV
        MMDIT_HIP(gemm_2(proj_base(d, 3 * H, H, ws.h, ws.h8, ws.sh, MMDIT_EPI_BIAS, ws.qkv, 3 * H),
                         group(0, Lt, w->txt.qkv), group(Lt, Li, w->img.qkv), s));
        // a4: QK-RMSNorm + RoPE + relayout
        MMDIT_HIP(launch_qknorm_rope(ws.qkv, 3 * H, L, d->heads, d->head_dim, Lt,
                                     w->txt.q_norm, w->txt.k_norm, w->img.q_norm, w->img.k_norm, rope,
                                     d->rms_eps, LP, ws.q, ws.k, ws.vt, s));
    }
    // a5: joint attention (fp8 blocks: on e4m3 q, k, v^T, the q/k scales
    // bounded by both streams' norm scales)
    if (fp8) {
        const uint16_t* qn1 = w->img.q_norm ? w->img.q_norm : w->txt.q_norm;
        const uint16_t* kn1 = w->img.k_norm ? w->img.k_norm : w->txt.k_norm;
        if (H % 256 == 0)   // q, k codes came from the QKV epilogue; v^T needs its per-channel maxima
            MMDIT_HIP(launch_quantize_vt_fp8(ws.vt, d->heads, d->head_dim, LP, ws.vt8, ws.sv, s));
        else
            MMDIT_HIP(launch_quantize_attention_fp8(ws.q, ws.k, ws.vt, d->heads, d->head_dim, LP, w->txt.q_norm,
                                                    qn1, w->txt.k_norm, kn1, ws.q8, ws.k8, ws.vt8, ws.sv, ws.exps,
                                                    s));
        MMDIT_HIP(launch_attention_fp8(ws.q8, ws.k8, ws.vt8, ws.sv, ws.exps, d->heads, L, d->head_dim, LP, ws.o, H,
                                       s));
    } else {
        MMDIT_HIP(launch_attention(ws.q, ws.k, ws.vt, d->heads, L, d->head_dim, LP, ws.o, H, s));
    }
    // a6: out projection + gated residual
    if (fp8) MMDIT_HIP(quant_rows(ws.o, L, H, ws.o8, ws.so, s));
    {
        GemmArgs g = proj_base(d, H, H, ws.o, ws.o8, ws.so, MMDIT_EPI_GATE_RESID, x_out, H);
        g.resid = x_in;
        g.ldr = H;
        MMDIT_HIP(gemm_2(g, group(0, Lt, w->txt.proj, mt + 2 * H), group(Lt, Li, w->img.proj, mi + 2 * H), s));
    }
    // a7: LN2 + modulate
    MMDIT_HIP(launch_ln_modulate(x_out, L, H, Lt, mt + 3 * H, mt + 4 * H, mi + 3 * H, mi + 4 * H,
                                 d->ln_eps, ws.h, s, fp8 ? ws.h8 : nullptr, fp8 ? ws.sh : nullptr));
    // a8: fc1 + GELU (or SwiGLU: fc1 rows [gate | up], hidden = SiLU(gate) * up)
    {
        const int epi = d->mlp_act == MMDIT_ACT_SWIGLU ? MMDIT_EPI_SWIGLU : MMDIT_EPI_BIAS_GELU;
        MMDIT_HIP(gemm_2(proj_base(d, mlp_cols(d), H, ws.h, ws.h8, ws.sh, epi, ws.a, M),
                         group(0, Lt, w->txt.fc1), group(Lt, Li, w->img.fc1), s));
    }
    if (fp8) MMDIT_HIP(quant_rows(ws.a, L, M, ws.a8, ws.sa, s));
    // a9: fc2 + gated residual
    {
        GemmArgs g = proj_base(d, H, M, ws.a, ws.a8, ws.sa, MMDIT_EPI_GATE_RESID, x_out, H);
        g.resid = x_out;
        g.ldr = H;
        MMDIT_HIP(gemm_2(g, group(0, Lt, w->txt.fc2, mt + 5 * H), group(Lt, Li, w->img.fc2, mi + 5 * H), s));
    }
    return MMDIT_OK;
}

int run_single(const mmdit_dims* d, const mmdit_single_weights* w, const float* vec, const float* rope,
               const float* x_in, float* x_out, const SingleWs& ws, hipStream_t s,
               const float* premod = nullptr) {
    const int L = seq_len(d), H = d->hidden, M = d->mlp_hidden;
    const int dt = d->weight_dtype, LP = padded_len(d);
    const float* m = premod ? premod : ws.mod;
    if (!premod) MMDIT_HIP(gemv(vec, H, w->mod, 3 * H, dt, 1, 0, ws.mod, s));
    const bool fp8 = dt == MMDIT_FP8;
    MMDIT_HIP(launch_ln_modulate(x_in, L, H, 0, m, m + H, m, m + H, d->ln_eps, ws.h, s,
                                 fp8 ? ws.h8 : nullptr, fp8 ? ws.sh : nullptr));
    {
        const bool fused = H % 256 == 0;
        const bool swiglu = d->mlp_act == MMDIT_ACT_SWIGLU;
        const int epi = fused ? (swiglu ? EPI_SPLIT_SWIGLU_ATTN : EPI_SPLIT_GELU_ATTN)
                              : (swiglu ? MMDIT_EPI_SPLIT_SWIGLU : MMDIT_EPI_SPLIT_GELU);
        GemmArgs g = proj_base(d, 3 * H + mlp_cols(d), H, ws.h, ws.h8, ws.sh, epi, ws.qkv, 3 * H);
        g.split_n = 3 * H;
        g.out2 = ws.cat;
        g.ldo2 = H + M;
        g.out2_col = H;
        GemmGroup g0 = group(0, L, w->linear1);
        if (fused) {
            // q|k|v columns: QK-RMSNorm, RoPE and the attention layouts in the
            // epilogue (as in the double block); the MLP columns as before
            g.q_out = ws.q;
            g.k_out = ws.k;
            g.vt_out = ws.vt;
            g.l_pad = LP;
            g.head_dim = d->head_dim;
            g.rope = rope;
            g.rms_eps = d->rms_eps;
            g0.qn = w->q_norm;
            g0.kn = w->k_norm;
            if (fp8) set_fp8_qk(g, d, ws.q8, ws.k8, ws.exps, w->q_norm, w->q_norm, w->k_norm, w->k_norm);
        }
        MMDIT_HIP(gemm_1(g, g0, s));
        if (fused) MMDIT_HIP(launch_zero_attn_pad(ws.q, ws.k, ws.vt, d->heads, d->head_dim, L, LP, s));
        else
            MMDIT_HIP(launch_qknorm_rope(ws.qkv, 3 * H, L, d->heads, d->head_dim, L, w->q_norm, w->k_norm,
                                         w->q_norm, w->k_norm, rope, d->rms_eps, LP, ws.q, ws.k, ws.vt, s));
    }
    if (fp8) {
        if (H % 256 == 0)   // q, k codes came from linear1's epilogue
            MMDIT_HIP(launch_quantize_vt_fp8(ws.vt, d->heads, d->head_dim, LP, ws.vt8, ws.sv, s));
        else
            MMDIT_HIP(launch_quantize_attention_fp8(ws.q, ws.k, ws.vt, d->heads, d->head_dim, LP, w->q_norm,
                                                    nullptr, w->k_norm, nullptr, ws.q8, ws.k8, ws.vt8, ws.sv,
                                                    ws.exps, s));
        MMDIT_HIP(launch_attention_fp8(ws.q8, ws.k8, ws.vt8, ws.sv, ws.exps, d->heads, L, d->head_dim, LP, ws.cat,
                                       H + M, s));
    } else {
        MMDIT_HIP(launch_attention(ws.q, ws.k, ws.vt, d->heads, L, d->head_dim, LP, ws.cat, H + M, s));
    }
    if (fp8) MMDIT_HIP(quant_rows(ws.cat, L, H + M, ws.cat8, ws.sc, s));
    {
        GemmArgs g = proj_base(d, H, H + M, ws.cat, ws.cat8, ws.sc, MMDIT_EPI_GATE_RESID, x_out, H);
        g.resid = x_in;
        g.ldr = H;
        MMDIT_HIP(gemm_1(g, group(0, L, w->linear2, m + 2 * H), s));
    }
    return MMDIT_OK;
}

int run_time_embed(const mmdit_dims* d, const mmdit_model* m, float t, float guidance, float* vec,
                   float* emb, float* tmp, hipStream_t s) {
    const int H = d->hidden, dt = d->weight_dtype;
    MMDIT_HIP(launch_time_and_guidance_embedding(t, guidance, emb, s));
    MMDIT_HIP(gemv(emb, 256, m->time_in[0], H, dt, 0, 0, tmp, s));
    MMDIT_HIP(gemv(tmp, H, m->time_in[1], H, dt, 1, 0, vec, s));
    if (d->guidance_embed) {
        MMDIT_HIP(gemv(emb + 256, 256, m->guid_in[0], H, dt, 0, 0, tmp + H, s));
        MMDIT_HIP(gemv(tmp + H, H, m->guid_in[1], H, dt, 1, 1, vec, s));
    }
    return MMDIT_OK;
}

// Per-step modulation layout: [double b: txt 6H | img 6H] for every double
// block, then [single b: 3H], then the final layer's [shift | scale] (2H).
size_t mod_floats(const mmdit_dims* d) {
    const size_t H = d->hidden;
    return (size_t)d->n_double * 12 * H + (size_t)d->n_single * 3 * H + 2 * H;
}
size_t mod_double_off(const mmdit_dims* d, int b) { return (size_t)b * 12 * d->hidden; }
size_t mod_single_off(const mmdit_dims* d, int b) {
    return (size_t)d->n_double * 12 * d->hidden + (size_t)b * 3 * d->hidden;
}
size_t mod_final_off(const mmdit_dims* d) { return mod_floats(d) - 2 * (size_t)d->hidden; }

struct ModBatchWs {
    float* emb;      // [512]
    float* tmp;      // [2H]
    float* vecs;     // [n_steps, H]
    uint16_t* a16;   // [n_steps, H] fp16 SiLU(vec)
};

ModBatchWs carve_modbatch(const mmdit_dims* d, int n_steps, Carver& c) {
    const size_t H = d->hidden;
    ModBatchWs w;
    w.emb = c.take<float>(512);
    w.tmp = c.take<float>(2 * H);
    w.vecs = c.take<float>((size_t)n_steps * H);
    w.a16 = c.take<uint16_t>((size_t)n_steps * H);
    return w;
}

// Weight type of the step's patch embedding, final projection and batched
// modulation GEMMs: their activation operands stay 16-bit, so an fp8 model's
// weights there are decoded to fp16 in registers (fp8 weight-only).
int io_wtype(int dt) { return dt == MMDIT_FP8 ? WT_FP8_W16A : dt; }

int model_ok(const mmdit_dims* d, const mmdit_model* m) {
    if (!m) return MMDIT_E_NULL;
    if (d->in_channels < 64 || d->in_channels % 64 != 0) return MMDIT_E_SHAPE;
    if (d->n_double < 0 || d->n_single < 0) return MMDIT_E_SHAPE;
    const int dt = d->weight_dtype;
    MMDIT_TRY(check_linear(m->img_in, dt));
    for (int i = 0; i < 2; ++i) {
        MMDIT_TRY(check_linear(m->time_in[i], dt));
        if (d->guidance_embed) MMDIT_TRY(check_linear(m->guid_in[i], dt));
    }
    MMDIT_TRY(check_linear(m->final_mod, dt));
    MMDIT_TRY(check_linear(m->final_out, dt));
    if (d->n_double > 0 && !m->doubles) return MMDIT_E_NULL;
    if (d->n_single > 0 && !m->singles) return MMDIT_E_NULL;
    for (int i = 0; i < d->n_double; ++i) MMDIT_TRY(double_weights_ok(&m->doubles[i], dt));
    for (int i = 0; i < d->n_single; ++i) MMDIT_TRY(single_weights_ok(&m->singles[i], dt));
    return MMDIT_OK;
}

// The step after validation. premod: this step's modulation (mod_floats
// layout) or null to compute the conditioning and every modulation here.
int run_step(const mmdit_dims* d, const mmdit_model* m, const float* premod, float* latent, const float* txt,
             const float* rope, float t_cur, float t_next, float guidance, const StepWs& sw, hipStream_t s) {
    const int Lt = d->txt_len, Li = d->img_len, H = d->hidden, C = d->in_channels, dt = d->weight_dtype;
    const int Ln = Li - d->ref_len;   // noisy image rows; the rest is the reference latent
    if (!premod) MMDIT_TRY(run_time_embed(d, m, t_cur, guidance, sw.vec, sw.emb, sw.tmp, s));
    // x = [txt | img_in(latent)] (reference rows included)
    MMDIT_HIP(launch_copy_f32(sw.x, txt, (int64_t)Lt * H, s));
    {
        const int64_t n = (int64_t)Li * C;
        int64_t blocks = (n + 255) / 256;
        if (blocks > 4096) blocks = 4096;
        hipLaunchKernelGGL(f32_to_f16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, latent, sw.z16, n);
        MMDIT_HIP(hipGetLastError());
        GemmArgs g = gemm_base(H, C, io_wtype(dt), sw.z16, C, MMDIT_EPI_BIAS_F32, sw.x + (size_t)Lt * H, H);
        MMDIT_HIP(gemm_1(g, group(0, Li, m->img_in), s));
    }
    Carver cb(sw.blocks);
    const DoubleWs dws = carve_double(d, cb);
    Carver cs(sw.blocks);
    const SingleWs sws = carve_single(d, cs);
    for (int i = 0; i < d->n_double; ++i)
        MMDIT_TRY(run_double(d, &m->doubles[i], sw.vec, rope, sw.x, sw.x, dws, s,
                             premod ? premod + mod_double_off(d, i) : nullptr));
    for (int i = 0; i < d->n_single; ++i)
        MMDIT_TRY(run_single(d, &m->singles[i], sw.vec, rope, sw.x, sw.x, sws, s,
                             premod ? premod + mod_single_off(d, i) : nullptr));
    // final layer on the noisy image rows, fused with the Euler update
    const float* fmod = premod ? premod + mod_final_off(d) : sw.fmod;
    if (!premod) MMDIT_HIP(gemv(sw.vec, H, m->final_mod, 2 * H, dt, 1, 0, sw.fmod, s));
    MMDIT_HIP(launch_ln_modulate(sw.x + (size_t)Lt * H, Ln, H, 0, fmod, fmod + H, fmod, fmod + H, d->ln_eps,
                                 dws.h, s));
    {
        GemmArgs g = gemm_base(C, H, io_wtype(dt), dws.h, H, MMDIT_EPI_EULER, latent, C);
        g.alpha = t_next - t_cur;
        MMDIT_HIP(gemm_1(g, group(0, Ln, m->final_out), s));
    }
    return MMDIT_OK;
}

}  // namespace

// ======================================================================== ABI
extern "C" {

int mmdit_abi_version(void) { return MMDIT_ABI_VERSION; }

const char* mmdit_status_string(int st) {
    switch (st) {
        case MMDIT_OK: return "ok";
        case MMDIT_E_NULL: return "null pointer";
        case MMDIT_E_ALIGN: return "pointer or stride not 16-byte aligned";
        case MMDIT_E_SHAPE: return "unsupported or inconsistent sizes";
        case MMDIT_E_DTYPE: return "bad weight dtype or missing int8 scales";
        case MMDIT_E_WORKSPACE: return "workspace too small";
        case MMDIT_E_HIP: return "kernel launch failed";
        case MMDIT_E_ARG: return "invalid argument";
        case MMDIT_E_SCRATCH: return "sizes exceed the fixed scratch of the no-allocation entry point";
        default: return "unknown status";
    }
}

size_t mmdit_workspace_bytes(const mmdit_dims* d, int kind) {
    if (check_dims(d) != MMDIT_OK) return 0;
    Carver c(nullptr);
    if (kind == MMDIT_WS_DOUBLE) carve_double(d, c);
    else if (kind == MMDIT_WS_SINGLE) carve_single(d, c);
    else if (kind == MMDIT_WS_STEP) carve_step(d, c);
    else return 0;
    return c.off;
}

int mmdit_block_forward(const mmdit_dims* d, const mmdit_double_weights* w, const float* vec,
                        const float* rope, const float* x_in, float* x_out, void* ws, size_t ws_bytes,
                        hipStream_t s) {
    MMDIT_TRY(check_dims(d));
    MMDIT_TRY(double_weights_ok(w, d->weight_dtype));
    MMDIT_TRY(check_ptr(vec));
    MMDIT_TRY(check_ptr(rope));
    MMDIT_TRY(check_ptr(x_in));
    MMDIT_TRY(check_ptr(x_out));
    MMDIT_TRY(check_ptr(ws));
    Carver c(ws);
    const DoubleWs dw = carve_double(d, c);
    if (ws_bytes < c.off) return MMDIT_E_WORKSPACE;
    return run_double(d, w, vec, rope, x_in, x_out, dw, s);
}

int mmdit_single_block_forward(const mmdit_dims* d, const mmdit_single_weights* w, const float* vec,
                               const float* rope, const float* x_in, float* x_out, void* ws,
                               size_t ws_bytes, hipStream_t s) {
    MMDIT_TRY(check_dims(d));
    MMDIT_TRY(single_weights_ok(w, d->weight_dtype));
    MMDIT_TRY(check_ptr(vec));
    MMDIT_TRY(check_ptr(rope));
    MMDIT_TRY(check_ptr(x_in));
    MMDIT_TRY(check_ptr(x_out));
    MMDIT_TRY(check_ptr(ws));
    Carver c(ws);
    const SingleWs sw = carve_single(d, c);
    if (ws_bytes < c.off) return MMDIT_E_WORKSPACE;
    return run_single(d, w, vec, rope, x_in, x_out, sw, s);
}

int mmdit_denoise_step(const mmdit_dims* d, const mmdit_model* m, float* latent, const float* txt,
                       const float* rope, float t_cur, float t_next, float guidance, void* ws,
                       size_t ws_bytes, hipStream_t s) {
    MMDIT_TRY(check_dims(d));
    MMDIT_TRY(model_ok(d, m));
    MMDIT_TRY(check_ptr(latent));
    MMDIT_TRY(check_ptr(txt));
    MMDIT_TRY(check_ptr(rope));
    MMDIT_TRY(check_ptr(ws));
    if (!std::isfinite(t_cur) || !std::isfinite(t_next) || !std::isfinite(guidance)) return MMDIT_E_ARG;
    Carver c(ws);
    const StepWs sw = carve_step(d, c);
    if (ws_bytes < c.off) return MMDIT_E_WORKSPACE;
    return run_step(d, m, nullptr, latent, txt, rope, t_cur, t_next, guidance, sw, s);
}

size_t mmdit_modulation_floats(const mmdit_dims* d) {
    if (check_dims(d) != MMDIT_OK || d->n_double < 0 || d->n_single < 0) return 0;
    return mod_floats(d);
}

size_t mmdit_modulation_workspace_bytes(const mmdit_dims* d, int n_steps) {
    if (check_dims(d) != MMDIT_OK || n_steps < 1 || n_steps > MMDIT_MAX_BATCH_STEPS) return 0;
    Carver c(nullptr);
    carve_modbatch(d, n_steps, c);
    return c.off;
}

}  // extern "C"

namespace {

// Arguments of a modulation batch, apart from its workspace.
int modbatch_args_ok(const mmdit_dims* d, const mmdit_model* m, const float* t, int n_steps, float guidance,
                     const float* mod) {
    MMDIT_TRY(check_dims(d));
    MMDIT_TRY(model_ok(d, m));
    if (!t) return MMDIT_E_NULL;
    if (n_steps < 1 || n_steps > MMDIT_MAX_BATCH_STEPS) return MMDIT_E_SHAPE;
    for (int i = 0; i < n_steps; ++i)
        if (!std::isfinite(t[i])) return MMDIT_E_ARG;
    if (!std::isfinite(guidance)) return MMDIT_E_ARG;
    MMDIT_TRY(check_ptr(mod));
    return MMDIT_OK;
}

// The modulation batch after validation, on a workspace of at least
// mmdit_modulation_workspace_bytes(d, n_steps) bytes. Every workspace byte it
// reads it has written first in the same call.
int run_modbatch(const mmdit_dims* d, const mmdit_model* m, const float* t, int n_steps, float guidance,
                 float* mod, void* ws, hipStream_t s) {
    Carver c(ws);
    const ModBatchWs w = carve_modbatch(d, n_steps, c);
    const int H = d->hidden, dt = d->weight_dtype;
    const int ld = (int)mod_floats(d);
    // conditioning vectors of every step, then SiLU(vec) as the fp16 operand
    for (int i = 0; i < n_steps; ++i)
        MMDIT_TRY(run_time_embed(d, m, t[i], guidance, w.vecs + (size_t)i * H, w.emb, w.tmp, s));
    MMDIT_HIP(launch_silu_to_f16(w.vecs, w.a16, (int64_t)n_steps * H, s));
    // one GEMM per modulation linear over all steps: each weight is read once
    auto mod_gemm = [&](const mmdit_linear& l, int n, size_t off) -> int {
        GemmArgs g = gemm_base(n, H, io_wtype(dt), w.a16, H, MMDIT_EPI_BIAS_F32, mod + off, ld);
        MMDIT_HIP(gemm_1(g, group(0, n_steps, l), s));
        return MMDIT_OK;
    };
    for (int b = 0; b < d->n_double; ++b) {
        MMDIT_TRY(mod_gemm(m->doubles[b].txt.mod, 6 * H, mod_double_off(d, b)));
        MMDIT_TRY(mod_gemm(m->doubles[b].img.mod, 6 * H, mod_double_off(d, b) + 6 * (size_t)H));
    }
    for (int b = 0; b < d->n_single; ++b) MMDIT_TRY(mod_gemm(m->singles[b].mod, 3 * H, mod_single_off(d, b)));
    MMDIT_TRY(mod_gemm(m->final_mod, 2 * H, mod_final_off(d)));
    return MMDIT_OK;
}

// ---- the scratch of mmdit_modulation_batch_noalloc: a fixed device array
// in the library's code object, one copy per GPU, held until the process
// ends. Host code never uses the array's name as an address: the name is a
// host-side stand-in, so each device's address is looked up once, with that
// device current, and kept.
__device__ __align__(256) char scratch[MMDIT_NOALLOC_SCRATCH_BYTES];

constexpr int kScratchDevices = 64;

// This device's address of `scratch` (null on failure).
void* scratch_on_current_device() {
    static std::atomic<void*> addr[kScratchDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return nullptr;
    void* p = addr[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        addr[dev].store(p, std::memory_order_release);   // a racing thread stores the same address
    }
    return p;
}

}  // namespace

extern "C" {

int mmdit_modulation_batch(const mmdit_dims* d, const mmdit_model* m, const float* t, int n_steps,
                           float guidance, float* mod, void* ws, size_t ws_bytes, hipStream_t s) {
    MMDIT_TRY(modbatch_args_ok(d, m, t, n_steps, guidance, mod));
    MMDIT_TRY(check_ptr(ws));
    Carver c(nullptr);
    carve_modbatch(d, n_steps, c);
    if (ws_bytes < c.off) return MMDIT_E_WORKSPACE;
    return run_modbatch(d, m, t, n_steps, guidance, mod, ws, s);
}

int mmdit_modulation_batch_noalloc(const mmdit_dims* d, const mmdit_model* m, const float* t, int n_steps,
                                   float guidance, float* mod, hipStream_t s) {
    MMDIT_TRY(modbatch_args_ok(d, m, t, n_steps, guidance, mod));
    Carver c(nullptr);
    carve_modbatch(d, n_steps, c);
    if (c.off > MMDIT_NOALLOC_SCRATCH_BYTES) return MMDIT_E_SCRATCH;
    void* ws = scratch_on_current_device();
    if (!ws) return MMDIT_E_HIP;
    return run_modbatch(d, m, t, n_steps, guidance, mod, ws, s);
}

int mmdit_denoise_step_premod(const mmdit_dims* d, const mmdit_model* m, const float* mod, float* latent,
                              const float* txt, const float* rope, float t_cur, float t_next, void* ws,
                              size_t ws_bytes, hipStream_t s) {
    MMDIT_TRY(check_dims(d));
    MMDIT_TRY(model_ok(d, m));
    MMDIT_TRY(check_ptr(mod));
    MMDIT_TRY(check_ptr(latent));
    MMDIT_TRY(check_ptr(txt));
    MMDIT_TRY(check_ptr(rope));
    MMDIT_TRY(check_ptr(ws));
    if (!std::isfinite(t_cur) || !std::isfinite(t_next)) return MMDIT_E_ARG;
    Carver c(ws);
    const StepWs sw = carve_step(d, c);
    if (ws_bytes < c.off) return MMDIT_E_WORKSPACE;
    return run_step(d, m, mod, latent, txt, rope, t_cur, t_next, 0.f, sw, s);
}

int mmdit_rope_table(const mmdit_dims* d, const int32_t* ids, float* rope, hipStream_t s) {
    MMDIT_TRY(check_dims(d));
    MMDIT_TRY(check_ptr(ids));
    MMDIT_TRY(check_ptr(rope));
    MMDIT_HIP(launch_rope_table(ids, seq_len(d), d->head_dim, d->rope_axes[0], d->rope_axes[1],
                                d->rope_axes[2], d->rope_theta, rope, s));
    return MMDIT_OK;
}

// ------------------------------------------------------------ kernel entries
int mmdit_k_ln_modulate(const float* x, int rows, int hidden, int split, const float* shift0,
                        const float* scale0, const float* shift1, const float* scale1, float eps,
                        mmdit_bf16* out, hipStream_t s) {
    if (rows < 0 || hidden < 64 || hidden % 64 != 0 || hidden > 4096) return MMDIT_E_SHAPE;
    if (!(eps > 0.f)) return MMDIT_E_ARG;
    MMDIT_TRY(check_ptr(x));
    MMDIT_TRY(check_ptr(out));
    MMDIT_TRY(check_ptr(shift0));
    MMDIT_TRY(check_ptr(scale0));
    if (split < rows) {
        MMDIT_TRY(check_ptr(shift1));
        MMDIT_TRY(check_ptr(scale1));
    }
    MMDIT_HIP(launch_ln_modulate(x, rows, hidden, split, shift0, scale0, shift1 ? shift1 : shift0,
                                 scale1 ? scale1 : scale0, eps, out, s));
    return MMDIT_OK;
}

int mmdit_k_qknorm_rope(const mmdit_bf16* qkv, int ld, int seq, int heads, int head_dim, int split,
                        const mmdit_bf16* qn0, const mmdit_bf16* kn0, const mmdit_bf16* qn1,
                        const mmdit_bf16* kn1, const float* rope, float eps, int l_pad,
                        mmdit_bf16* q_out, mmdit_bf16* k_out, mmdit_bf16* vt_out, hipStream_t s) {
    if (head_dim != 64 && head_dim != 128) return MMDIT_E_SHAPE;
    if (seq < 1 || heads < 1 || ld < 3 * heads * head_dim || ld % 8 != 0) return MMDIT_E_SHAPE;
    if (l_pad < seq || l_pad % 64 != 0) return MMDIT_E_SHAPE;
    if (!(eps > 0.f)) return MMDIT_E_ARG;
    for (const void* p : {(const void*)qkv, (const void*)qn0, (const void*)kn0, (const void*)rope,
                          (const void*)q_out, (const void*)k_out, (const void*)vt_out})
        MMDIT_TRY(check_ptr(p));
    if (split < seq) {
        MMDIT_TRY(check_ptr(qn1));
        MMDIT_TRY(check_ptr(kn1));
    }
    MMDIT_HIP(launch_qknorm_rope(qkv, ld, seq, heads, head_dim, split, qn0, kn0, qn1 ? qn1 : qn0,
                                 kn1 ? kn1 : kn0, rope, eps, l_pad, q_out, k_out, vt_out, s));
    return MMDIT_OK;
}

int mmdit_k_attention(const mmdit_bf16* q, const mmdit_bf16* k, const mmdit_bf16* vt, int heads, int seq,
                      int head_dim, int l_pad, mmdit_bf16* out, int ldo, hipStream_t s) {
    if (head_dim != 64 && head_dim != 128) return MMDIT_E_SHAPE;
    if (seq < 1 || heads < 1 || l_pad < seq || l_pad % 64 != 0 || l_pad >= (1 << 24)) return MMDIT_E_SHAPE;
    if (ldo < heads * head_dim || ldo % 8 != 0) return MMDIT_E_SHAPE;
    for (const void* p : {(const void*)q, (const void*)k, (const void*)vt, (const void*)out})
        MMDIT_TRY(check_ptr(p));
    MMDIT_HIP(launch_attention(q, k, vt, heads, seq, head_dim, l_pad, out, ldo, s));
    return MMDIT_OK;
}

int mmdit_k_quantize_attention_fp8(const mmdit_bf16* q, const mmdit_bf16* k, const mmdit_bf16* vt, int heads,
                                   int head_dim, int l_pad, const mmdit_bf16* q_norm0, const mmdit_bf16* q_norm1,
                                   const mmdit_bf16* k_norm0, const mmdit_bf16* k_norm1, uint8_t* q8, uint8_t* k8,
                                   uint8_t* vt8, float* v_scale, int32_t* exps, hipStream_t s) {
    if (head_dim != 64 && head_dim != 128) return MMDIT_E_SHAPE;
    if (heads < 1 || l_pad < 64 || l_pad % 64 != 0 || l_pad >= (1 << 24)) return MMDIT_E_SHAPE;
    for (const void* p : {(const void*)q, (const void*)k, (const void*)vt, (const void*)q_norm0, (const void*)k_norm0,
                          (const void*)q8, (const void*)k8, (const void*)vt8, (const void*)v_scale, (const void*)exps})
        MMDIT_TRY(check_ptr(p));
    MMDIT_HIP(launch_quantize_attention_fp8(q, k, vt, heads, head_dim, l_pad, q_norm0, q_norm1, k_norm0, k_norm1, q8,
                                            k8, vt8, v_scale, exps, s));
    return MMDIT_OK;
}

int mmdit_k_attention_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* vt8, const float* v_scale,
                          const int32_t* exps, int heads, int seq, int head_dim, int l_pad, mmdit_f16* out, int ldo,
                          hipStream_t s) {
    if (head_dim != 64 && head_dim != 128) return MMDIT_E_SHAPE;
    if (seq < 1 || heads < 1 || l_pad < seq || l_pad % 64 != 0 || l_pad >= (1 << 24)) return MMDIT_E_SHAPE;
    if (ldo < heads * head_dim || ldo % 8 != 0) return MMDIT_E_SHAPE;
    for (const void* p : {(const void*)q8, (const void*)k8, (const void*)vt8, (const void*)v_scale, (const void*)exps,
                          (const void*)out})
        MMDIT_TRY(check_ptr(p));
    MMDIT_HIP(launch_attention_fp8(q8, k8, vt8, v_scale, exps, heads, seq, head_dim, l_pad, out, ldo, s));
    return MMDIT_OK;
}

int mmdit_k_gemm(const mmdit_gemm* g, hipStream_t s) {
    if (!g) return MMDIT_E_NULL;
    if (g->m < 1 || g->n < 64 || g->n % 64 != 0 || g->k < 64 || g->k % 64 != 0) return MMDIT_E_SHAPE;
    if (g->lda < g->k || g->lda % 8 != 0) return MMDIT_E_SHAPE;
    // per-lane operand offsets are 32-bit within a 256-row tile (SwiGLU: a
    // tile's up rows lie n/2 weight rows past its gate rows)
    {
        const uint64_t es = g->weight_dtype == MMDIT_FP8 ? 1 : 2;
        const uint64_t w_rows = g->epilogue == MMDIT_EPI_SWIGLU || g->epilogue == MMDIT_EPI_SPLIT_SWIGLU
                                    ? (uint64_t)g->n / 2 + 256 : 256;
        if (256 * (uint64_t)g->lda * es + (uint64_t)g->k * es >= (1ull << 32) ||
            w_rows * (uint64_t)g->k * es + (uint64_t)g->k * es >= (1ull << 32))
            return MMDIT_E_SHAPE;
    }
    if (!dtype_ok(g->weight_dtype) && g->weight_dtype != MMDIT_FP8) return MMDIT_E_DTYPE;
    if (g->epilogue < MMDIT_EPI_BIAS || g->epilogue > MMDIT_EPI_SPLIT_SWIGLU) return MMDIT_E_ARG;
    if (g->weight_dtype == MMDIT_FP8) {
        // fp8 codes for A too: 128 k per stage, rows 16-byte aligned, a row scale
        if (g->k % 128 != 0 || g->lda % 16 != 0) return MMDIT_E_SHAPE;
        if (g->epilogue == MMDIT_EPI_SWIGLU || g->epilogue == MMDIT_EPI_SPLIT_SWIGLU) return MMDIT_E_ARG;
        MMDIT_TRY(check_ptr(g->a_scale));
    }
    MMDIT_TRY(check_ptr(g->a));
    MMDIT_TRY(check_linear(g->w, g->weight_dtype));
    MMDIT_TRY(check_ptr(g->out));
    const bool f32out = g->epilogue == MMDIT_EPI_GATE_RESID || g->epilogue == MMDIT_EPI_BIAS_F32 ||
                        g->epilogue == MMDIT_EPI_EULER;
    const bool split = g->epilogue == MMDIT_EPI_SPLIT_GELU || g->epilogue == MMDIT_EPI_SPLIT_SWIGLU;
    const int ncols = split ? g->split_n : g->epilogue == MMDIT_EPI_SWIGLU ? g->n / 2 : g->n;
    if (g->ldo < ncols || g->ldo % (f32out ? 4 : 8) != 0) return MMDIT_E_SHAPE;
    if (g->epilogue == MMDIT_EPI_GATE_RESID) {
        MMDIT_TRY(check_ptr(g->gate));
        MMDIT_TRY(check_ptr(g->resid));
        if (g->ldr < g->n || g->ldr % 4 != 0) return MMDIT_E_SHAPE;
    }
    if (g->epilogue == MMDIT_EPI_SWIGLU && g->n % 256 != 0) return MMDIT_E_SHAPE;
    if (split) {
        const int q = g->epilogue == MMDIT_EPI_SPLIT_SWIGLU ? 256 : 64;   // SwiGLU tiles never straddle
        if (g->split_n < 0 || g->split_n > g->n || g->split_n % q != 0 || (g->n - g->split_n) % q != 0)
            return MMDIT_E_SHAPE;
        const int n2 = g->epilogue == MMDIT_EPI_SPLIT_SWIGLU ? (g->n - g->split_n) / 2 : g->n - g->split_n;
        MMDIT_TRY(check_ptr(g->out2));
        if (g->out2_col < 0 || g->out2_col % 8 != 0 || g->ldo2 % 8 != 0 || g->ldo2 < g->out2_col + n2)
            return MMDIT_E_SHAPE;
    }
    GemmArgs a = gemm_base(g->n, g->k, g->weight_dtype, g->a, g->lda, g->epilogue, g->out, g->ldo);
    a.resid = g->resid;
    a.ldr = g->ldr;
    a.split_n = g->split_n;
    a.out2 = g->out2;
    a.ldo2 = g->ldo2;
    a.out2_col = g->out2_col;
    a.alpha = g->alpha;
    a.a_scale = g->a_scale;
    MMDIT_HIP(gemm_1(a, group(0, g->m, g->w, g->gate), s));
    return MMDIT_OK;
}

int mmdit_quantize_fp8_rows(const void* x, int x_dtype, int rows, int cols, int ldx, uint8_t* codes, int ldc,
                            float* scales, hipStream_t s) {
    if (x_dtype != MMDIT_BF16 && x_dtype != MMDIT_F16) return MMDIT_E_DTYPE;
    if (rows < 0 || cols < 16 || cols % 16 != 0 || ldx < cols || ldx % 8 != 0 || ldc < cols || ldc % 16 != 0)
        return MMDIT_E_SHAPE;
    MMDIT_TRY(check_ptr(x));
    MMDIT_TRY(check_ptr(codes));
    MMDIT_TRY(check_ptr(scales));
    MMDIT_HIP(launch_quantize_fp8_rows(static_cast<const uint16_t*>(x), x_dtype == MMDIT_BF16, rows, cols, ldx,
                                       codes, ldc, scales, s));
    return MMDIT_OK;
}

int mmdit_k_gemv(const float* x, int k, const mmdit_linear* w, int n, int weight_dtype, int silu_input,
                 int accumulate, float* out, hipStream_t s) {
    if (!w) return MMDIT_E_NULL;
    if (k < 64 || k % 64 != 0 || n < 1 || k > 4096) return MMDIT_E_SHAPE;
    if (!dtype_ok(weight_dtype)) return MMDIT_E_DTYPE;
    MMDIT_TRY(check_ptr(x));
    MMDIT_TRY(check_linear(*w, weight_dtype));
    MMDIT_TRY(check_ptr(out));
    MMDIT_HIP(gemv(x, k, *w, n, weight_dtype, silu_input != 0, accumulate != 0, out, s));
    return MMDIT_OK;
}

int mmdit_k_time_embed(const mmdit_dims* d, const mmdit_model* m, float t, float guidance, float* vec,
                       void* ws, size_t ws_bytes, hipStream_t s) {
    MMDIT_TRY(check_dims(d));
    if (!m) return MMDIT_E_NULL;
    for (int i = 0; i < 2; ++i) {
        MMDIT_TRY(check_linear(m->time_in[i], d->weight_dtype));
        if (d->guidance_embed) MMDIT_TRY(check_linear(m->guid_in[i], d->weight_dtype));
    }
    MMDIT_TRY(check_ptr(vec));
    MMDIT_TRY(check_ptr(ws));
    if (ws_bytes < 4 * (512 + 2 * (size_t)d->hidden)) return MMDIT_E_WORKSPACE;
    float* emb = static_cast<float*>(ws);
    return run_time_embed(d, m, t, guidance, vec, emb, emb + 512, s);
}

int mmdit_weights_to_f16(const mmdit_bf16* src, mmdit_f16* dst, size_t count, hipStream_t s) {
    MMDIT_TRY(check_ptr(src));
    MMDIT_TRY(check_ptr(dst));
    const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
    if (count > 0 && a < b + 2 * count && b < a + 2 * count) return MMDIT_E_ARG;
    MMDIT_HIP(launch_bf16_to_f16(src, dst, count, s));
    return MMDIT_OK;
}

int mmdit_k_euler(float* z, const float* v, int64_t n, float dt, hipStream_t s) {
    if (n < 0) return MMDIT_E_SHAPE;
    MMDIT_TRY(check_ptr(z));
    MMDIT_TRY(check_ptr(v));
    MMDIT_HIP(launch_euler(z, v, n, dt, s));
    return MMDIT_OK;
}

}  // extern "C"
