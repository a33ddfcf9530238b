/*
 * mmdit.h - C ABI of the MI355X (gfx950) MM-DiT block library, libmmdit.so.
 *
 * The library runs the bf16 forward pass of a multimodal diffusion-transformer
 * block (double-stream and single-stream) and one flow-matching Euler denoise
 * step, as hand-written HIP kernels. The operations follow the Luminal blog
 * "Reducing image generation cost with..." (sections "Flux.2 Klein 9B", "The
 * AMD MI300X pipeline" and "What the compiler found on its own") and the
 * flux-amd-rocm benchmarks page (28 Euler steps, guidance 3.5, int8
 * weight-only linears).
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Pointers to tensors are DEVICE pointers, except the structs themselves
 *   (mmdit_dims, mmdit_linear, weight structs, mmdit_gemm), which live in host
 *   memory and hold device pointers.
 * - Every device pointer must be 16-byte aligned; every row stride (ld*)
 *   is in elements and must keep 16-byte alignment of every row.
 * - bf16 tensors are raw IEEE bfloat16 bit patterns (mmdit_bf16), fp16
 *   tensors raw IEEE binary16 bit patterns (mmdit_f16); fp32 is IEEE
 *   binary32. Matrices are row-major.
 * - Precision: weights are bf16 (or int8 codes with fp32 scales); the
 *   residual stream, conditioning vector, latent and RoPE table are fp32;
 *   attention runs bf16 MFMA on bf16 q, k, v; the activation operands of the
 *   projections (LayerNorm outputs, attention output, GELU hidden) are fp16,
 *   and each weight fragment is converted to fp16 in registers (exact for
 *   bf16 weights of magnitude >= 2^-14 and for int8 codes); every sum
 *   accumulates in fp32.
 * - Range: fp16 holds magnitudes up to 65504. An activation operand beyond
 *   that (a LayerNorm output with |(1 + scale)| or |shift| in the
 *   thousands, an attention output of a value row beyond it, a GELU hidden
 *   beyond it) is stored as +-inf (IEEE conversion, no saturation), so the
 *   block output turns non-finite rather than silently wrong. The residual
 *   stream, vec and the latent are fp32 and have no such limit. (DiT
 *   activations after LayerNorm are O(10); the synthetic workloads stay far
 *   inside the range.)
 * - The caller owns every buffer (weights, activations, tables, workspace).
 *   The library allocates nothing and frees nothing. The only values it
 *   keeps between calls are per-device caches of device properties (the
 *   compute-unit count, whether a kernel's LDS limit is set), thread-safe
 *   and never affecting results; calls on different streams with distinct
 *   workspaces may overlap.
 * - Every call only enqueues work on `stream` and returns; nothing is
 *   synchronised. Outputs are defined once the stream has reached the work.
 * - Arguments are validated before anything is enqueued: on a non-zero
 *   status nothing was launched. A device fault surfaces at the caller's next
 *   synchronisation. Status MMDIT_E_HIP reports a failed launch.
 * - Results are deterministic: the same inputs, sizes and stream order give
 *   bit-identical outputs (no atomics, fixed reduction order).
 * - Batch is 1: a "sequence" is one image with its prompt.
 */
#ifndef MMDIT_H
#define MMDIT_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MMDIT_ABI_VERSION 3

/* raw bfloat16 bits */
typedef uint16_t mmdit_bf16;
/* raw IEEE binary16 bits */
typedef uint16_t mmdit_f16;

/* ------------------------------------------------------------------ status */
enum mmdit_status {
    MMDIT_OK = 0,
    MMDIT_E_NULL = 1,      /* a required pointer is NULL */
    MMDIT_E_ALIGN = 2,     /* a pointer or row stride breaks 16-byte alignment */
    MMDIT_E_SHAPE = 3,     /* unsupported or inconsistent sizes */
    MMDIT_E_DTYPE = 4,     /* unknown weight dtype, or int8 weights without scales */
    MMDIT_E_WORKSPACE = 5, /* workspace too small */
    MMDIT_E_HIP = 6,       /* a kernel launch failed */
    MMDIT_E_ARG = 7,       /* another invalid argument (unknown enum value) */
    MMDIT_E_SCRATCH = 8    /* sizes need more than the fixed scratch of a
                              no-allocation entry point */
};

enum mmdit_weight_dtype {
    MMDIT_BF16 = 0, /* weights are bf16 [out, in] */
    MMDIT_INT8 = 1, /* weights are int8 codes [out, in] with fp32 scale [out]:
                       W = diag(scale) * codes (flux-amd-rocm benchmarks page:
                       int8 weight-only linears) */
    MMDIT_F16 = 2,  /* weights are fp16 [out, in]: bf16 weights re-encoded once
                       by mmdit_weights_to_f16. The matrix cores take both
                       operands in one format and the activation operands are
                       fp16, so the bf16 path converts every weight fragment
                       in registers on every use; this format does it once.
                       Same rounding, so results are bit-identical to
                       MMDIT_BF16 with the bf16 originals */
    MMDIT_FP8 = 3   /* OCP fp8 e4m3 codes [out, in] with an fp32 scale per output
                       channel: W = diag(scale) * decode(codes). GEMMs only
                       (mmdit_k_gemm): the activation operand is fp8 e4m3 too,
                       with an fp32 scale per row (mmdit_gemm.a_scale), and the
                       product runs on the fp8 matrix cores (SGLang-AMD,
                       "Architecture Deep Dive": fp8 on CDNA). Codes and scales
                       come from mmdit_quantize_fp8_rows. The block entries
                       accept it for GELU MLPs: every projection's activation
                       operand is quantised per token right before its GEMM
                       (LayerNorm outputs, attention output, GELU hidden), and
                       the attention runs on e4m3 q, k, v and probabilities
                       (mmdit_k_quantize_attention_fp8 and
                       mmdit_k_attention_fp8, with the q/k scales bounded by
                       the block's q/k norm scales); the residual stream is
                       unchanged. The
                       step entries accept it too: the blocks as above; the
                       embedders, modulations, patch embedding and final
                       projection keep 16-bit (fp32 for the GEMVs)
                       activations against the fp8 weights, decoded exactly
                       in registers (fp8 weight-only) */
};

/* ------------------------------------------------------------------ sizes */
/*
 * Sizes of one model. H = heads * head_dim.
 *   head_dim in {64, 128}; hidden a multiple of 64 up to 4096; mlp_hidden a
 *   multiple of 64 up to 65536; txt_len + img_len up to 2^20;
 *   rope_axes[] even, summing to head_dim (axial RoPE over (t, h, w));
 *   txt_len >= 1, img_len >= 1; in_channels a multiple of 64 (64 for FLUX);
 *   n_double / n_single: block counts of a whole model (denoise step only).
 * The joint sequence holds txt_len text tokens, then img_len image tokens.
 */
typedef struct mmdit_dims {
    int32_t txt_len;
    int32_t img_len;
    int32_t hidden;
    int32_t heads;
    int32_t head_dim;
    int32_t mlp_hidden;
    int32_t in_channels;
    int32_t rope_axes[3];
    float rope_theta;   /* 1e4 */
    float ln_eps;       /* LayerNorm epsilon, 1e-6 */
    float rms_eps;      /* RMSNorm epsilon, 1e-6 */
    int32_t weight_dtype; /* enum mmdit_weight_dtype */
    int32_t n_double;
    int32_t n_single;
    int32_t mlp_act;        /* enum mmdit_mlp_act */
    int32_t guidance_embed; /* 1: vec = MLP_t(emb(t)) + MLP_g(emb(guidance)) (FLUX.1-dev);
                               0: vec = MLP_t(emb(t)), guid_in unused (guidance-free,
                               step-distilled Flux.2 Klein, "Flux.2 Klein 9B" section) */
    int32_t ref_len;        /* image editing ("Flux.2 Klein 9B" section: the image-to-image
                               pipeline): the last ref_len of the img_len image-stream
                               tokens are the encoded reference image. They take part in
                               every block; the denoise step reads them and updates only
                               the first img_len - ref_len rows. 0 <= ref_len < img_len */
} mmdit_dims;

/* Activation of the MLP (double-stream fc1, single-stream linear1 MLP part) */
enum mmdit_mlp_act {
    MMDIT_ACT_GELU_TANH = 0, /* fc1 [M, H]; hidden = GELU_tanh(fc1(h)) */
    MMDIT_ACT_SWIGLU = 1     /* fc1 [2M, H] rows [gate | up]; hidden = SiLU(gate) * up
                                (Luminal blog, "What the compiler found on its own":
                                the fused SwiGLU activation of Flux.2 Klein). Needs
                                hidden % 256 == 0 and mlp_hidden % 128 == 0 */
};

/* ------------------------------------------------------------------ weights */
/*
 * One linear layer y = x W^T + b. w: [out, in] row-major, bf16 bits or int8
 * codes per the dtype in use; scale: fp32 [out] (int8 only, else ignored);
 * bias: bf16 [out] (required).
 */
typedef struct mmdit_linear {
    const void* w;
    const float* scale;
    const mmdit_bf16* bias;
} mmdit_linear;

/*
 * One stream of a double-stream block ("Flux.2 Klein 9B" section: each stream
 * has its own projections, norm and feed-forward network).
 *   mod  [6H, H]: SiLU(vec) -> [shift1 | scale1 | gate1 | shift2 | scale2 | gate2]
 *   qkv  [3H, H]: columns [q | k | v], each head-major (column h*D + d)
 *   proj [H, H], fc1 [M, H] (SwiGLU: [2M, H], rows [gate | up]), fc2 [H, M]
 *   q_norm, k_norm: bf16 [D] RMSNorm scales of this stream
 */
typedef struct mmdit_stream_weights {
    mmdit_linear mod, qkv, proj, fc1, fc2;
    const mmdit_bf16* q_norm;
    const mmdit_bf16* k_norm;
} mmdit_stream_weights;

typedef struct mmdit_double_weights {
    mmdit_stream_weights txt, img;
} mmdit_double_weights;

/*
 * Single-stream block: one set of weights over the joint sequence.
 *   mod     [3H, H]:   [shift | scale | gate]
 *   linear1 [3H+M, H]: columns [q | k | v | mlp]
 *           (SwiGLU: [3H+2M, H], columns [q | k | v | gate | up])
 *   linear2 [H, H+M]:  input [attention | GELU(mlp)] (SwiGLU: [attention | SiLU(gate) * up])
 */
typedef struct mmdit_single_weights {
    mmdit_linear mod, linear1, linear2;
    const mmdit_bf16* q_norm;
    const mmdit_bf16* k_norm;
} mmdit_single_weights;

/*
 * A whole denoiser. img_in [H, C]; time_in / guid_in: Linear(256 -> H), SiLU,
 * Linear(H -> H) of the sinusoidal embedding (guid_in is not read when
 * dims->guidance_embed is 0); final_mod [2H, H] ->
 * [shift | scale]; final_out [C, H]. doubles / singles: HOST arrays of
 * n_double / n_single block weight structs.
 */
typedef struct mmdit_model {
    mmdit_linear img_in;
    mmdit_linear time_in[2];
    mmdit_linear guid_in[2];
    mmdit_linear final_mod;
    mmdit_linear final_out;
    const mmdit_double_weights* doubles;
    const mmdit_single_weights* singles;
} mmdit_model;

/* ------------------------------------------------------------------ blocks */
enum mmdit_workspace_kind {
    MMDIT_WS_DOUBLE = 0,
    MMDIT_WS_SINGLE = 1,
    MMDIT_WS_STEP = 2
};

/* Bytes of workspace the given call needs for these sizes (0 on bad sizes). */
size_t mmdit_workspace_bytes(const mmdit_dims* dims, int kind);

/*
 * Double-stream block forward (Luminal blog, "Flux.2 Klein 9B" and "What the
 * compiler found on its own"): per stream, modulation of SiLU(vec),
 * LayerNorm + modulate, QKV projection, per-head RMSNorm of q and k; over the
 * joint sequence, axial RoPE and softmax attention without a mask; per
 * stream, output projection with gated residual, LayerNorm + modulate, GELU
 * (or SwiGLU, dims->mlp_act) MLP with gated residual.
 *   vec:   fp32 [H] conditioning vector
 *   rope:  fp32 [L, D/2, 2] (cos, sin) per rotated pair (mmdit_rope_table)
 *   x_in:  fp32 [L, H] joint residual stream, text rows first
 *   x_out: fp32 [L, H]; may alias x_in
 *   ws:    device workspace of at least mmdit_workspace_bytes(MMDIT_WS_DOUBLE)
 */
int mmdit_block_forward(const mmdit_dims* dims, const mmdit_double_weights* w,
                        const float* vec, const float* rope,
                        const float* x_in, float* x_out,
                        void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Single-stream block forward: modulation, LayerNorm + modulate, linear1
 * (q|k|v|mlp), RMSNorm + RoPE on q and k, attention, linear2 over
 * [attention | GELU(mlp)] (or [attention | SiLU(gate) * up]), gated residual.
 * Arguments as mmdit_block_forward.
 */
int mmdit_single_block_forward(const mmdit_dims* dims, const mmdit_single_weights* w,
                               const float* vec, const float* rope,
                               const float* x_in, float* x_out,
                               void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * One flow-matching Euler denoise step (flux-amd-rocm benchmarks page:
 * FLUX.1-dev, guidance 3.5; Luminal blog, "The AMD MI300X pipeline": the
 * latent is integrated in fp32):
 *   vec = MLP_t(emb(t_cur)) + MLP_g(emb(guidance)), emb = [cos | sin] of
 *   1000*t times 128 geometric frequencies (max period 1e4); without the
 *   guidance term when dims->guidance_embed is 0 (guidance is then unused);
 *   x = [txt | img_in(latent)]; n_double double blocks; n_single single
 *   blocks; v = final_out(LayerNorm(x_img) * (1 + scale) + shift) on the
 *   first img_len - ref_len image rows; latent += (t_next - t_cur) * v there.
 *   latent: fp32 [img_len, in_channels]; the first img_len - ref_len rows are
 *           updated in place, the last ref_len rows (the reference image of
 *           an edit) are only read
 *   txt:    fp32 [txt_len, H] text states
 *   rope:   fp32 [L, D/2, 2]
 *   dims->weight_dtype selects bf16, fp16 or int8 weights for every linear.
 */
int mmdit_denoise_step(const mmdit_dims* dims, const mmdit_model* model,
                       float* latent, const float* txt, const float* rope,
                       float t_cur, float t_next, float guidance,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Modulation of every block for many denoise steps at once. The conditioning
 * vector depends only on the step's time (and the guidance value), not on
 * the latent, so the modulation of all blocks for all steps of a sampling
 * run is known before the first step; computed here as one GEMM per
 * modulation linear over all steps, each weight is read once per run instead
 * of once per step (Luminal blog, "Where the time goes on the MI300X": the
 * glue kernels; the modulations are 226 MB of weights per FLUX double block).
 *   t:   HOST array of n_steps step times (1 <= n_steps <= MMDIT_MAX_BATCH_STEPS)
 *   mod: fp32 [n_steps, mmdit_modulation_floats(dims)]; row i holds, for step
 *        i: per double block [txt 6H | img 6H], then per single block [3H],
 *        then the final layer's [shift | scale] (2H), chunk orders as in the
 *        weight structs
 *   ws:  at least mmdit_modulation_workspace_bytes(dims, n_steps)
 * The conditioning vectors are computed in fp32 as in mmdit_denoise_step;
 * SiLU(vec) enters the matrix cores as fp16 (the per-step path keeps it fp32
 * in its GEMV), a relative rounding of at most 2^-11 per element.
 */
#define MMDIT_MAX_BATCH_STEPS 256
size_t mmdit_modulation_floats(const mmdit_dims* dims);
size_t mmdit_modulation_workspace_bytes(const mmdit_dims* dims, int n_steps);
int mmdit_modulation_batch(const mmdit_dims* dims, const mmdit_model* model,
                           const float* t, int n_steps, float guidance,
                           float* mod, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * mmdit_modulation_batch without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation). Its scratch is a fixed device
 * array inside the library, MMDIT_NOALLOC_SCRATCH_BYTES per GPU, held from
 * the library's load until the process ends; this entry point allocates and
 * frees nothing. Sizes whose workspace (mmdit_modulation_workspace_bytes)
 * exceeds it are rejected with MMDIT_E_SCRATCH before anything is enqueued:
 * 4 MiB covers n_steps * hidden up to about 650 K (256 steps up to hidden
 * 2560; 28 steps at any hidden size the library accepts). The result is
 * bit-identical to mmdit_modulation_batch's. Every call on one GPU shares
 * that GPU's array: calls that overlap on one GPU (other streams, other host
 * threads) race and must be ordered by the caller. Each call writes every
 * scratch byte before it reads it, so no clearing is needed.
 */
#define MMDIT_NOALLOC_SCRATCH_BYTES (4u << 20)
int mmdit_modulation_batch_noalloc(const mmdit_dims* dims, const mmdit_model* model,
                                   const float* t, int n_steps, float guidance,
                                   float* mod, hipStream_t stream);

/*
 * mmdit_denoise_step with the modulation given: mod is this step's row of
 * mmdit_modulation_batch (fp32 [mmdit_modulation_floats(dims)], device). No
 * conditioning vector and no modulation GEMV is computed; everything else is
 * as in mmdit_denoise_step (same workspace, MMDIT_WS_STEP). The launch
 * sequence is fixed for fixed dims, pointers and times, and enqueues no
 * memory fills, so a caller may capture it in a HIP graph.
 */
int mmdit_denoise_step_premod(const mmdit_dims* dims, const mmdit_model* model,
                              const float* mod, float* latent, const float* txt,
                              const float* rope, float t_cur, float t_next,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * RoPE table from axial position ids: ids int32 [L, 3] (t, h, w) on the
 * device; rope fp32 [L, D/2, 2]. Pair p of the head dim belongs to axis a
 * (consecutive segments of rope_axes[0], [1], [2] dims); its j-th pair in
 * that axis turns by ids[l][a] * theta^(-2j / rope_axes[a]) (Luminal blog,
 * "What the compiler found on its own": cosine and sine tables).
 */
int mmdit_rope_table(const mmdit_dims* dims, const int32_t* ids, float* rope,
                     hipStream_t stream);

const char* mmdit_status_string(int status);
int mmdit_abi_version(void);

/*
 * Re-encode bf16 weights as fp16 for MMDIT_F16 (a load-time step, like the
 * upload of the weights). Each value is rounded to nearest-even fp16: exact
 * for magnitudes in [2^-14, 65504]; smaller ones round to fp16 subnormals
 * (steps of 2^-24); magnitudes >= 65520 become infinities. These are the
 * values the bf16 path feeds its matrix cores.
 *   src: bf16 [count]; dst: fp16 [count]; both 16-byte aligned, may not overlap.
 * Errors: E_NULL, E_ALIGN; count 0 enqueues nothing.
 */
int mmdit_weights_to_f16(const mmdit_bf16* src, mmdit_f16* dst, size_t count, hipStream_t stream);

/* ------------------------------------------------------------------ kernels */
/*
 * Single-kernel entry points, used by the block calls and exposed for tests
 * and per-kernel measurement. Same conventions as above.
 */

/*
 * LayerNorm (no affine, biased variance) + adaLN modulate ("What the compiler
 * found on its own": a mean, a subtraction, a reciprocal square root, then a
 * scale and a shift): out = LN(x) * (1 + scale) + shift.
 *   x: fp32 [rows, hidden]; rows < split take (shift0, scale0), the others
 *   (shift1, scale1), each fp32 [hidden]; out: fp16 [rows, hidden].
 */
int mmdit_k_ln_modulate(const float* x, int rows, int hidden, int split,
                        const float* shift0, const float* scale0,
                        const float* shift1, const float* scale1,
                        float eps, mmdit_f16* out, hipStream_t stream);

/*
 * Per-head RMSNorm of q and k, then axial RoPE, then relayout for attention
 * ("What the compiler found on its own": square, sum, reciprocal square root,
 * multiply; partner gather and multiply-add against cos/sin tables).
 *   qkv: bf16 [seq_len, ld]; q at columns [0, H), k at [H, 2H), v at [2H, 3H)
 *   rows < split use (q_norm0, k_norm0), the others (q_norm1, k_norm1): bf16 [D]
 *   rope: fp32 [seq_len, D/2, 2]
 *   q_out, k_out: bf16 [heads, l_pad, D]; vt_out: bf16 [heads, D, l_pad], V
 *   transposed (keys along the row) with the keys of every aligned group of 16
 *   stored in the order 0-3, 8-11, 4-7, 12-15 (the two middle quads swapped),
 *   so that each 16-byte chunk holds the 8 keys one matrix-core lane needs.
 *   l_pad: a multiple of 64, >= seq_len; rows [seq_len, l_pad) are written as 0.
 */
int mmdit_k_qknorm_rope(const mmdit_bf16* qkv, int ld, int seq_len, int heads, int head_dim,
                        int split, const mmdit_bf16* q_norm0, const mmdit_bf16* k_norm0,
                        const mmdit_bf16* q_norm1, const mmdit_bf16* k_norm1,
                        const float* rope, float eps, int l_pad,
                        mmdit_bf16* q_out, mmdit_bf16* k_out, mmdit_bf16* vt_out,
                        hipStream_t stream);

/*
 * Softmax attention without a mask (Luminal blog, "What the compiler found on
 * its own" and "The AMD MI300X pipeline": fused, tiled softmax(QK^T)V).
 *   q, k: bf16 [heads, l_pad, D]; vt: bf16 [heads, D, l_pad] in the
 *   quad-swapped key order written by mmdit_k_qknorm_rope (zero beyond
 *   seq_len); l_pad a multiple of 64 and below 2^24; scale 1/sqrt(D).
 *   out: fp16 [seq_len, ldo], head h at columns [h*D, (h+1)*D).
 */
int mmdit_k_attention(const mmdit_bf16* q, const mmdit_bf16* k, const mmdit_bf16* vt,
                      int heads, int seq_len, int head_dim, int l_pad,
                      mmdit_f16* out, int ldo, hipStream_t stream);

/*
 * fp8 attention (SGLang-AMD, "Architecture Deep Dive": fp8 quantisation on
 * the CDNA stack; the attention products of the Luminal blog's "What the
 * compiler found on its own" on the fp8 matrix cores). Two calls:
 *
 * mmdit_k_quantize_attention_fp8: q, k (bf16 [heads, l_pad, D]) and vt (bf16
 *   [heads, D, l_pad], the order mmdit_k_qknorm_rope writes) to OCP e4m3:
 *   - q and k at one power-of-two scale per tensor, 2^eq and 2^ek: e is the
 *     smallest integer with 2^e >= fl32(fl32(sqrt(D)/448) * max|g|), max over
 *     the RMSNorm scales q_norm0/q_norm1 (k_norm0/k_norm1; the second of each
 *     may be NULL, as for a single-stream block). After RMSNorm and RoPE
 *     every element is at most sqrt(D) max|g| in magnitude, so no code
 *     overflows; inputs that are not RMS-normalised with these scales may
 *     exceed 448 and are outside this contract.
 *     q8, k8: codes [heads, l_pad, D] (1 byte each); exps: int32[2] = (eq, ek).
 *   - vt with one fp32 scale per channel (row of vt): v_scale[h*D + d] =
 *     max over the row of |v| / 448, code = e4m3(v / scale) (both in fp32;
 *     0 for an all-zero row). vt8: codes [heads, D, l_pad] with the keys of
 *     each 64-key tile in the order of the fp8 kernel's operand slots: slot
 *     32g + 16s + 4a + b holds key 32s + 8a + 4g + b (g, s < 2; a, b < 4).
 *   Rounding to nearest even throughout; the caller owns every buffer.
 *
 * mmdit_k_attention_fp8: O = softmax attention on those codes:
 *   logits in log2 units t = (q8 . k8) 2^(eq+ek) log2(e) / sqrt(D); the
 *   exponentials p = 2^(t - M + 8) with M the smallest integer at or above
 *   the row's maximum t, so p lies in [0, 256]; the value product takes the
 *   e4m3 codes of p, the row sum the fp32 p:
 *   O[i, h*D + d] = v_scale[h*D + d] * sum_j e4m3(p_ij) v8[j, d] / sum_j p_ij.
 *   (The kernel tracks M tile by tile; M being an integer makes the codes the
 *   same as against the final M up to exact powers of two.) out: fp16
 *   [seq_len, ldo]. Shapes as for mmdit_k_attention.
 */
int mmdit_k_quantize_attention_fp8(const mmdit_bf16* q, const mmdit_bf16* k, const mmdit_bf16* vt,
                                   int heads, int head_dim, int l_pad,
                                   const mmdit_bf16* q_norm0, const mmdit_bf16* q_norm1,
                                   const mmdit_bf16* k_norm0, const mmdit_bf16* k_norm1,
                                   uint8_t* q8, uint8_t* k8, uint8_t* vt8, float* v_scale,
                                   int32_t* exps, hipStream_t stream);
int mmdit_k_attention_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* vt8,
                          const float* v_scale, const int32_t* exps,
                          int heads, int seq_len, int head_dim, int l_pad,
                          mmdit_f16* out, int ldo, hipStream_t stream);

/* GEMM epilogues (bias is always added first: y = acc * s + b, s = 1 for bf16) */
enum mmdit_epilogue {
    MMDIT_EPI_BIAS = 0,       /* out bf16 [m, ldo] = y (q, k, v for attention) */
    MMDIT_EPI_BIAS_GELU = 1,  /* out fp16 = GELU_tanh(y) (MLP hidden) */
    MMDIT_EPI_GATE_RESID = 2, /* out fp32 = resid + gate[n] * y (out may alias resid) */
    MMDIT_EPI_SPLIT_GELU = 3, /* columns n < split_n: out bf16 [m, ldo] col n = y;
                                 n >= split_n: out2 fp16 [m, ldo2] col
                                 out2_col + n - split_n = GELU_tanh(y) */
    MMDIT_EPI_BIAS_F32 = 4,   /* out fp32 [m, ldo] = y */
    MMDIT_EPI_EULER = 5,      /* out fp32 [m, ldo] += alpha * y (the Euler update) */
    MMDIT_EPI_SWIGLU = 6,     /* gated MLP (Luminal blog, "What the compiler found on
                                 its own": fused SwiGLU of Flux.2 Klein). W rows are
                                 [gate (n/2) | up (n/2)]; out fp16 [m, ldo] col f =
                                 SiLU(y_f) * y_{n/2+f}, f < n/2. n a multiple of 256 */
    MMDIT_EPI_SPLIT_SWIGLU = 7 /* columns n < split_n: out bf16 [m, ldo] col n = y;
                                 the rest, [gate (M) | up (M)] with M = (n - split_n)/2:
                                 out2 fp16 [m, ldo2] col out2_col + f = SiLU(gate_f) * up_f.
                                 split_n and n - split_n multiples of 256 */
};

/*
 * out = epilogue(A W^T): A fp16 [m, k] (row stride lda), W = w.w [n, k] bf16,
 * fp16 or int8 (weight_dtype). k a multiple of 64, n a multiple of 64, m >= 1;
 * 256 * lda and (256 + n/2 for SwiGLU epilogues, else 256) * k, in bytes, below
 * 4 GiB (the kernel addresses each 256-row tile with 32-bit offsets from its
 * first row), else MMDIT_E_SHAPE.
 * bf16 and int8 weight fragments are converted to fp16 in registers (see
 * above);
 * accumulation in fp32; the int8 per-channel scale multiplies the fp32 sum.
 */
typedef struct mmdit_gemm {
    int32_t m, n, k;
    int32_t weight_dtype;
    const mmdit_f16* a;
    int32_t lda;
    mmdit_linear w;
    int32_t epilogue;
    void* out;
    int32_t ldo;
    const float* gate;  /* fp32 [n], GATE_RESID */
    const float* resid; /* fp32 [m, ldr], GATE_RESID */
    int32_t ldr;
    int32_t split_n;    /* SPLIT_GELU */
    void* out2;
    int32_t ldo2;
    int32_t out2_col;
    float alpha;        /* EULER */
    const float* a_scale; /* fp32 [m], MMDIT_FP8 only: row i of A is a_scale[i] * decode(a[i]) */
} mmdit_gemm;

/* With weight_dtype MMDIT_FP8, a holds fp8 e4m3 codes (lda in bytes, a
 * multiple of 16), k is a multiple of 128, w.scale and a_scale are required:
 * y[i][j] = a_scale[i] * w.scale[j] * sum_k decode(a[i][k]) decode(w[j][k]) + b[j]
 * (the fp8 products are exact and the sums accumulate in fp32). */
int mmdit_k_gemm(const mmdit_gemm* g, hipStream_t stream);

/*
 * Per-row fp8 quantisation (OCP e4m3, largest finite value 448): for each of
 * `rows` rows of x (16-bit floats, x_dtype MMDIT_BF16 or MMDIT_F16, row
 * stride ldx elements, `cols` values), scale = max|x| / 448 (fp32 division)
 * and code = e4m3(x / scale) (fp32 division, round to nearest even); an
 * all-zero row gets scale 0 and zero codes. Weights [out, in] quantised this
 * way get one scale per output channel; activations one per token.
 *   codes: fp8 [rows, ldc] (ldc bytes >= cols, a multiple of 16); scales: fp32 [rows]
 */
int mmdit_quantize_fp8_rows(const void* x, int x_dtype, int rows, int cols, int ldx,
                            uint8_t* codes, int ldc, float* scales, hipStream_t stream);

/*
 * out[n] (+)= W act(x) + b for one vector (modulation and embedder layers):
 *   x fp32 [k], k a multiple of 64 and <= 4096; act = SiLU if silu_input else
 *   identity; W [n, k] bf16, fp16 or int8 (weight_dtype);
 *   accumulate: 0 writes out, 1 adds to it. out fp32 [n].
 */
int mmdit_k_gemv(const float* x, int k, const mmdit_linear* w, int n, int weight_dtype,
                 int silu_input, int accumulate, float* out, hipStream_t stream);

/*
 * Conditioning vector vec fp32 [H] = MLP_t(emb(t)) + MLP_g(emb(guidance)).
 * ws: device scratch of at least 4 * (512 + 2 * H) bytes.
 */
int mmdit_k_time_embed(const mmdit_dims* dims, const mmdit_model* model, float t,
                       float guidance, float* vec, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/* Euler update z[i] += dt * v[i], fp32, n elements. */
int mmdit_k_euler(float* z, const float* v, int64_t n, float dt, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MMDIT_H */
