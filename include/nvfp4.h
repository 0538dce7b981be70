/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) small-M NVFP4 W4A4 decode linear.
 *
 * The operation: "ReSET: Accurate Latency-Critical NVFP4 Reasoning via
 * Step-Aware Temperature Scaling", GitHub README, section "Core components",
 * item 2 (kernels/, nvfp4r): a decode linear y = x W^T for M <= 8 activation
 * rows in which both operands are NVFP4 (W4A4), computed by streaming the FP4
 * weights once and reusing every loaded weight for all M rows.  The arXiv
 * abstract states the same problem (small-M NVFP4 kernel for latency-critical
 * autoregressive decoding).  The same README's "Quantize a model to NVFP4"
 * section covers converting bf16 weights to NVFP4 offline.
 *
 * Number format (the pages name NVFP4 without defining it; the public NVFP4
 * layout is used): element = E2M1 code (OCP MX v1.0, 5.3.3), one E4M3 ("FN",
 * OCP OFP8) scale per 16 consecutive elements along K, one binary32 scale per
 * tensor.  x_hat = e2m1(code) * e4m3(scale) * gscale.
 *
 * Quantizer Q(X) for a bf16 tensor X [R][K] (every step binary32, round to
 * nearest even, no fused multiply-add, denormals kept):
 *   A = max|x| over the tensor;  gscale = A / 2688 (= 6 * 448), 1 if that is 0
 *   per 16-block: a = max|x|; sigma = a / (gscale * 6);
 *     scale byte = E4M3 round-to-nearest-even of sigma, saturating at 448;
 *     T = e4m3(scale) * gscale;  r = (T == 0) ? 0 : 1 / T;
 *     code = E2M1 round-to-nearest-even of x * r, saturating at 6, sign bit
 *     taken from x (so -0 gives code 0x8).
 *
 * Canonical layouts (row-major, used for activations and for export):
 *   codes  [R][K/2]  byte i holds element 2i in bits 0..3, 2i+1 in bits 4..7
 *   scales [R][K/16] one E4M3 byte per block
 *
 * Device-tiled weight layout (layout version 1), padded to N_pad = 32 *
 * ceil(N/32) rows and K_pad = 256 * ceil(K/256) columns; padding holds code 0
 * and scale 0:
 *   codes:  1024-byte records, record (t, c) at byte (t * K_pad/64 + c) * 1024
 *           for row tile t (rows 32t..32t+31) and K chunk c (64 elements).
 *           Inside a record, the 16 bytes at 16 * l (l = 0..63) hold row
 *           32t + (l % 32), elements 64c + 32*(l / 32) + 0..31, packed as in
 *           the canonical layout.
 *   scales: 512-byte records, record (t, g) at byte (t * K_pad/256 + g) * 512
 *           for K group g (256 elements).  The 8 bytes at 8 * l hold the
 *           scales of row 32t + (l % 32), blocks 16g + 4q + 2*(l / 32) + b
 *           at byte 2q + b (q = 0..3, b = 0..1).
 *   So every 64-lane wavefront load of a record is one contiguous 1 KiB
 *   (codes) or 512 B (scales), and lane l's code bytes in chunk c are covered
 *   by its own scale bytes.
 *
 * Conventions:
 *   - Pointers are device pointers unless a comment says "host".  The caller
 *     owns every buffer; no entry point allocates device memory or
 *     synchronizes the device, except the stack object (nvfp4_stack_*), which
 *     allocates its activation buffers once at creation.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously; every call in the linear and
 *     quantization paths can be captured into a HIP graph.
 *   - Argument errors are detected on the host before any HIP call and
 *     return without enqueuing work.  A failing HIP call returns
 *     NVFP4_ERR_HIP; its hipError_t is kept per host thread
 *     (nvfp4_last_hip_error).  Device faults surface at the caller's next
 *     synchronization, as for any HIP kernel.
 *   - Inputs must be finite.  A tensor amax in (0, 2^-90) is outside the
 *     contract (1/T may overflow): codes are then unspecified, never a crash.
 */
#ifndef NVFP4_DECODE_LINEAR_H
#define NVFP4_DECODE_LINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment      */
  NVFP4_ERR_UNSUPPORTED = 2, /* M > 8, device is not gfx950, unknown option */
  NVFP4_ERR_NO_DEVICE = 3,   /* no HIP device visible                      */
  NVFP4_ERR_WORKSPACE = 4,   /* workspace smaller than required            */
  NVFP4_ERR_HIP = 5          /* a HIP runtime call failed                  */
} nvfp4_status;

typedef enum { NVFP4_OUT_F32 = 0, NVFP4_OUT_BF16 = 1 } nvfp4_out_dtype;

/* Runtime knobs (process-global, atomic).  Counterpart of the README's
 * "nvfp4r.configure(gemv_max_m=2)" / "nvfp4r.status()" (section "Run
 * benchmarks", the Python wiring example). */
typedef enum {
  NVFP4_OPT_GEMV_MAX_M = 0,   /* M <= value uses the VALU GEMV (M <= 3 only);
                                 larger M the FP4 MFMA one.  0..8, default 0
                                 (MFMA for every M, the faster one on
                                 gfx950).                                   */
  NVFP4_OPT_SPLIT_K = 1,      /* 0 = heuristic; s >= 1 forces s K-slices.  */
  NVFP4_OPT_CHUNKS_PER_WAVE = 2, /* 0 = heuristic; else 64-element K chunks
                                 each wavefront streams per row tile (multiple
                                 of 4).                                     */
  NVFP4_OPT_NONTEMPORAL = 3,  /* 1 (default) = stream weights with
                                 non-temporal loads; 0 = ordinary loads.   */
  NVFP4_OPT_WAVES = 4,        /* 0 = heuristic; else 4, 8 or 16 wavefronts
                                 per GEMV workgroup (one 32-row tile); the
                                 streaming kernels take at most 8 (more is
                                 clamped to 8), the split kernel 16.       */
  NVFP4_OPT_KERNEL = 5,       /* 0 = heuristic; 1 = persistent streaming
                                 VALU GEMV (whole K per workgroup; M <= 3
                                 and the activation must fit in LDS, else
                                 the split kernel runs); 2 = split-K VALU
                                 GEMV (one workgroup per tile and K slice);
                                 3 = persistent streaming GEMV with the dot
                                 on FP4 MFMA (falls back to split-K when the
                                 activation does not fit in LDS).          */
  NVFP4_OPT_SPIN_LIMIT = 6,   /* 0 = default; else the number of polls the
                                 activation quantizer makes for the other
                                 workgroups' maxima before computing the
                                 tensor amax on its own (same result; a low
                                 value exercises that path).               */
  NVFP4_OPT_GRID = 7,         /* 0 = heuristic (one streaming workgroup per
                                 CU); else at most this many streaming
                                 workgroups, 1..65536 (above 256 several may
                                 share a CU).                               */
  NVFP4_OPT_FUSE_QUANT = 8,   /* 1 (default): nvfp4_quantize_linear quantizes
                                 the activation inside the GEMV whenever it
                                 can; 0: always as two launches.           */
  NVFP4_OPT_HALF_TILES = 9,   /* MFMA streaming kernel on 16-row half tiles
                                 (16x16x128 MFMA, twice the work items): 0
                                 (default) = when 32-row tiles fill at most
                                 half the 256 workgroups, 1 = never, 2 =
                                 always (one K slice only).                */
  NVFP4_OPT_F32_SLICES = 10,  /* nvfp4_quantize_linear_f32 given a maxima
                                 record: 0 (default) = never use the K-slice
                                 plan (two launches when the activation does
                                 not fit one prologue), 1 = only then, 2 =
                                 always (where a slice plan exists).       */
  NVFP4_OPT_COUNT = 11
} nvfp4_option;

/* ABI version of this header (incremented on any signature change). */
int nvfp4_abi_version(void);

/* Version of the device-tiled weight layout described above (1). */
int nvfp4_layout_version(void);

/* Static, never-freed description of a status code. */
const char* nvfp4_status_string(nvfp4_status s);

/* hipError_t of the last failing HIP call on this host thread (0 if none). */
int nvfp4_last_hip_error(void);

/* Set / read a runtime knob.  Unknown option or out-of-range value:
 * NVFP4_ERR_UNSUPPORTED / NVFP4_ERR_INVALID_ARG.  `value` is a host pointer. */
nvfp4_status nvfp4_set_option(int opt, int64_t value);
nvfp4_status nvfp4_get_option(int opt, int64_t* value);

/* Bytes of the device-tiled codes and scales for an N x K weight (host
 * outputs).  N >= 1, K >= 16, K % 16 == 0. */
nvfp4_status nvfp4_weight_bytes(int64_t N, int64_t K, size_t* codes_bytes, size_t* scales_bytes);

/* Weight quantization, once per model load (README "Quantize a model to
 * NVFP4": bf16 checkpoint -> NVFP4).
 *   w_bf16   [N][ldw] bf16 bit patterns, ldw >= K, row r at w_bf16 + r*ldw
 *   w_codes  device-tiled codes  (nvfp4_weight_bytes bytes)
 *   w_scales device-tiled scales (nvfp4_weight_bytes bytes)
 *   w_gscale one float, written on the device
 * Enqueues four kernels (init, tensor amax, blocks, finalize). */
nvfp4_status nvfp4_quantize_weight(const uint16_t* w_bf16, int64_t N, int64_t K, int64_t ldw,
                                   uint8_t* w_codes, uint8_t* w_scales, float* w_gscale,
                                   void* stream);

/* The gate_up weight [2F][K] (rows [0, F) gate, [F, 2F) up) quantized as
 * nvfp4_quantize_weight would, into the interleaved row order the SiLU * mul
 * epilogue reads (nvfp4_quantize_linear_silu_mul): tiled row 32t + r holds
 * source row 16t + r for r < 16 and F + 16t + r - 16 for r >= 16, so each
 * 32-row tile carries the gate and up rows of the same 16 output columns.
 * The result is exactly nvfp4_quantize_weight of the rows in that order
 * (the tensor scale does not depend on row order).  F % 16 == 0; the rest
 * as for nvfp4_quantize_weight with N = 2F. */
nvfp4_status nvfp4_quantize_weight_gate_up(const uint16_t* w_bf16, int64_t F, int64_t K,
                                           int64_t ldw, uint8_t* w_codes, uint8_t* w_scales,
                                           float* w_gscale, void* stream);

/* Inverse of the tiling: device-tiled weight -> canonical row-major codes
 * [N][K/2] and scales [N][K/16] (for export and bit-exact checks). */
nvfp4_status nvfp4_unpack_weight(const uint8_t* w_codes, const uint8_t* w_scales, int64_t N,
                                 int64_t K, uint8_t* codes_rowmajor, uint8_t* scales_rowmajor,
                                 void* stream);

/* Workspace bytes nvfp4_quantize_act needs: 0 when one workgroup covers the
 * tensor (M * K <= 16384), else 16 (the record in which the workgroups
 * combine their maxima).  0 also for arguments nvfp4_quantize_act rejects. */
size_t nvfp4_act_workspace_bytes(int M, int64_t K);

/* Activation quantization, every decode step (W4A4: the activations reach
 * the linear as NVFP4).  One tensor scale over the whole M x K input.
 *   x_bf16   [M][ldx] bf16, 1 <= M <= 8, M * K <= 2^22, ldx >= K,
 *            ldx % 8 == 0, 16-byte aligned base
 *   x_codes  [M][K/2] canonical;  x_scales [M][K/16] canonical
 *   x_gscale one float, written on the device (never read back to the host)
 *   workspace nvfp4_act_workspace_bytes bytes, 16-byte aligned, zeroed once
 *            by nvfp4_workspace_init; each call leaves it zero again, so it
 *            may be the same memory as nvfp4_linear's workspace when the
 *            calls are ordered on one stream, but two calls that can run
 *            concurrently need distinct workspaces.
 * The tensor maximum is combined across workgroups inside the one kernel
 * (each polls for the others a bounded number of times and otherwise
 * computes it alone, so the call always terminates with the same result). */
nvfp4_status nvfp4_quantize_act(const uint16_t* x_bf16, int M, int64_t K, int64_t ldx,
                                uint8_t* x_codes, uint8_t* x_scales, float* x_gscale,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Activation quantization with a caller-supplied tensor scale (a static,
 * calibrated activation scale, as carried by checkpoints from an offline
 * NVFP4 conversion: the "ReSET" GitHub README, "Quantize a model to NVFP4").
 * The quantizer Q above with its first step replaced: gscale = *x_gscale
 * (read on the device) instead of amax / 2688; every block then follows the
 * same steps, so blocks whose sigma exceeds 448 saturate to scale 448 and
 * codes +-6.
 *   x_gscale  one device float, finite and > 0, not written; inputs with
 *             a / (6 * x_gscale) beyond the binary32 range are outside the
 *             contract (codes unspecified, never a crash)
 *   other arguments as for nvfp4_quantize_act (no workspace: no tensor
 *   maximum is combined across workgroups). */
nvfp4_status nvfp4_quantize_act_static(const uint16_t* x_bf16, int M, int64_t K, int64_t ldx,
                                       const float* x_gscale, uint8_t* x_codes, uint8_t* x_scales,
                                       void* stream);

/* nvfp4_quantize_linear with the static tensor scale of
 * nvfp4_quantize_act_static: y = linear(Q_static(x)), bit-identical to
 * nvfp4_quantize_act_static followed by nvfp4_linear with x_gscale as the
 * activation tensor scale (x_codes and x_scales are written).  One kernel
 * whenever nvfp4_quantize_linear would fuse (its prologue then takes no
 * tensor maximum).  Workspace: nvfp4_quantize_linear_workspace_bytes. */
nvfp4_status nvfp4_quantize_linear_static(int M, int64_t N, int64_t K, const uint16_t* x_bf16,
                                          int64_t ldx, const float* x_gscale,
                                          const uint8_t* w_codes, const uint8_t* w_scales,
                                          const float* w_gscale, void* y, int out_dtype,
                                          uint8_t* x_codes, uint8_t* x_scales, void* workspace,
                                          size_t workspace_bytes, void* stream);

/* Activation quantization and the decode linear in one call: the result is
 * bit-identical to nvfp4_quantize_act(x_bf16 -> x_codes, x_scales,
 * x_gscale) followed by nvfp4_linear on those outputs, which this call also
 * writes.  When the plan streams the weights on the MFMA kernel and M * K /
 * 16 <= 2048 (4096 with M >= 4, at most 4 (8) blocks per thread of the
 * plan's workgroup), a single kernel does both: every workgroup quantizes the
 * activation in its prologue (reading the bf16 input from L2) and workgroup
 * 0 writes the quantized copy, so the separate quantizer launch disappears;
 * otherwise (or with NVFP4_OPT_FUSE_QUANT = 0) the two launches run in
 * order.  Arguments as for nvfp4_quantize_act and nvfp4_linear; x_codes,
 * x_scales and x_gscale are outputs here.  The workspace must hold
 * nvfp4_quantize_linear_workspace_bytes(M, N, K): the larger of the two
 * calls' needs and at least 16 bytes (the same memory serves both; 0 only
 * for arguments the call rejects). */
size_t nvfp4_quantize_linear_workspace_bytes(int M, int64_t N, int64_t K);
nvfp4_status nvfp4_quantize_linear(int M, int64_t N, int64_t K, const uint16_t* x_bf16, int64_t ldx,
                                   const uint8_t* w_codes, const uint8_t* w_scales,
                                   const float* w_gscale, void* y, int out_dtype, uint8_t* x_codes,
                                   uint8_t* x_scales, float* x_gscale, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* The unweighted per-row RMS norm, the activation quantizer and the linear
 * in one call: y = linear(Q(h)) with h as for nvfp4_rmsnorm_quantize_act
 * (x_codes, x_scales, x_gscale and, if not NULL, h_out [M][K] binary32 are
 * written).  In one kernel when nvfp4_quantize_linear would fuse and the
 * activation fits 4 blocks per thread at any M (M * K / 16 <= 2048 with 8
 * wavefronts; at 8 per thread the fused norm measured slower than its own
 * launch); its workgroups then sum each row's squares in their own fixed
 * order (the same
 * in every workgroup and on every run, but not the standalone quantizer's,
 * so h may differ from nvfp4_rmsnorm_quantize_act's in the last bits; either
 * way the codes are exactly Q of the h that is written).  Otherwise
 * nvfp4_rmsnorm_quantize_act then nvfp4_linear.  K <= 32768; workspace as for
 * nvfp4_quantize_linear. */
nvfp4_status nvfp4_rmsnorm_quantize_linear(int M, int64_t N, int64_t K, const uint16_t* x_bf16,
                                           int64_t ldx, float eps, const uint8_t* w_codes,
                                           const uint8_t* w_scales, const float* w_gscale,
                                           void* y, int out_dtype, uint8_t* x_codes,
                                           uint8_t* x_scales, float* x_gscale, float* h_out,
                                           void* workspace, size_t workspace_bytes,
                                           void* stream);

/* Fused quantizers of the layer stack (one decode step of a decoder: the
 * end-to-end figure of the "ReSET" GitHub README, captioned under its
 * introduction, runs the NVFP4 linears of whole layers; the stack between
 * the linears is this library's stand-in for the parts of a layer that are
 * not linears).  Each computes a
 * binary32 h from a bf16 input and applies the activation quantizer Q above to
 * h (the tensor maximum over all M x K values of h; the quantizer steps are
 * the same, starting from binary32 instead of bf16 values):
 *   rmsnorm:  h[m][k] = x[m][k] * (1 / sqrt(mean_k(x[m][k]^2) + eps)), the
 *             sum of squares in binary32 in a fixed order, every other step
 *             one correctly rounded binary32 operation (unweighted RMS norm);
 *   silu_mul: h[m][k] = (g / (1 + exp(-g))) * u with g = gu[m][k], u =
 *             gu[m][K + k] (first half gate, second half up), exp from the
 *             device math library (within a few ulp), the rest correctly
 *             rounded binary32.
 *   x_bf16 / gu_bf16  [M][ld] bf16, 1 <= M <= 8, 16 <= K <= 32768, K % 16 == 0,
 *            ld >= K (rmsnorm) or >= 2K (silu_mul), ld % 8 == 0, 16-byte
 *            aligned base
 *   codes/scales/gscale as for nvfp4_quantize_act
 *   h_out    optional (NULL: not written) binary32 [M][K], 16-byte aligned:
 *            the h that was quantized
 *   workspace at least 16 bytes when M > 1 (the same zero-initialised record
 *            nvfp4_quantize_act uses; it is left zero).  Optional at M = 1.
 * rmsnorm: one workgroup per row; the rows' maxima are combined as in
 * nvfp4_quantize_act.  silu_mul: with a workspace (any M) the M * K / 16
 * blocks are spread over workgroups of 256 threads, one block per thread,
 * and their maxima combined the same way; without one (M = 1) a single
 * workgroup does the row.  Both give the same h and codes. */
nvfp4_status nvfp4_rmsnorm_quantize_act(const uint16_t* x_bf16, int M, int64_t K, int64_t ldx,
                                        float eps, uint8_t* x_codes, uint8_t* x_scales,
                                        float* x_gscale, float* h_out, void* workspace,
                                        size_t workspace_bytes, void* stream);
nvfp4_status nvfp4_silu_mul_quantize_act(const uint16_t* gu_bf16, int M, int64_t K, int64_t ldgu,
                                         uint8_t* x_codes, uint8_t* x_scales, float* x_gscale,
                                         float* h_out, void* workspace, size_t workspace_bytes,
                                         void* stream);

/* SiLU * mul fused into the gate_up projection, and the down projection fed
 * from its binary32 output (the layer step between the two linears, with no
 * separate quantizer launch: "ReSET" GitHub README, "Core components" item
 * 2, the W4A4 decode linear; the SiLU * mul step as in the stack above).
 *
 * A maxima record is NVFP4_AMAX_RECORD_WORDS uint32 words, 16-byte aligned:
 * word i holds the largest |h| (binary32 bit pattern, sign cleared) of the
 * h values one workgroup wrote, zero for unused words, so the tensor maximum
 * of h is the record's largest word.  It lets the consumer take the tensor
 * scale without a pass over h. */
#define NVFP4_AMAX_RECORD_WORDS 256

/* gate_up linear + SiLU * mul:
 *   g = bf16(y[m][j]), u = bf16(y[m][F + j]),  h[m][j] = silu(g) * u  (j < F)
 * with y the linear of Q(x) (rmsnorm = 0) or of Q(rmsnorm(x)) (rmsnorm = 1,
 * h of the norm as in nvfp4_rmsnorm_quantize_linear) with the gate_up weight
 * [2F][K] (rows [0, F) gate, [F, 2F) up), the bf16 rounding the one the
 * linear's bf16 output applies, and silu(g) * u the element operation of
 * nvfp4_silu_mul_quantize_act.  So h is bit-identical to the h_out of
 * nvfp4_silu_mul_quantize_act on g and u (gu_out).
 *   x_bf16   [M][ldx] bf16 as for nvfp4_quantize_linear; eps as for the RMS norm
 *   w_*      the gate_up weight from nvfp4_quantize_weight_gate_up (the
 *            interleaved row order); F % 16 == 0
 *   h        binary32 [M][ldh], ldh >= F, ldh % 4 == 0, 16-byte aligned
 *   h_amax   the maxima record of h (written whole)
 *   gu_out   optional (NULL: not written) bf16 [M][2F]: g and u as above
 *   x_codes, x_scales, x_gscale  the quantized activation (written)
 *   xh_out   optional binary32 [M][K]: the normalised input (rmsnorm = 1 only)
 *   workspace  at least 16 bytes when M > 1 (used only when the activation
 *            is quantized by its own launch first; left zero)
 * One kernel when the activation fits the GEMV's quantizing prologue (as for
 * nvfp4_quantize_linear), else the quantizer then the GEMV.  The GEMV runs
 * on whole 32-row tiles with one K slice (each tile holds both factors of
 * its 16 columns); NVFP4_ERR_UNSUPPORTED if no such plan fits. */
nvfp4_status nvfp4_quantize_linear_silu_mul(int M, int64_t F, int64_t K, const uint16_t* x_bf16,
                                            int64_t ldx, int rmsnorm, float eps,
                                            const uint8_t* w_codes, const uint8_t* w_scales,
                                            const float* w_gscale, float* h, int64_t ldh,
                                            uint32_t* h_amax, uint16_t* gu_out, uint8_t* x_codes,
                                            uint8_t* x_scales, float* x_gscale, float* xh_out,
                                            void* workspace, size_t workspace_bytes,
                                            void* stream);

/* The activation quantizer Q on a binary32 activation x_f32 [M][ldx] (ldx >=
 * K, ldx % 4 == 0, 16-byte aligned): the quantizer steps of
 * nvfp4_quantize_act starting from binary32 values.  x_amax: NULL, or the
 * maxima record of x_f32 written by its producer (then the tensor maximum is
 * read from it and no workspace is needed); without it the workspace holds
 * the 16-byte sync record of nvfp4_quantize_act. */
nvfp4_status nvfp4_quantize_act_f32(const float* x_f32, int M, int64_t K, int64_t ldx,
                                    const uint32_t* x_amax, uint8_t* x_codes, uint8_t* x_scales,
                                    float* x_gscale, void* workspace, size_t workspace_bytes,
                                    void* stream);

/* nvfp4_quantize_act_f32 and nvfp4_linear in one call (x_codes, x_scales,
 * x_gscale written).  One kernel when the activation fits the quantizing
 * prologue (M * K / 16 <= 4 blocks per thread of the plan's workgroup, and
 * <= 4096), on nvfp4_linear's own plan: y is then bit-identical to
 * nvfp4_linear on the written codes.  Otherwise the two launches (the
 * quantizer then nvfp4_linear), unless NVFP4_OPT_F32_SLICES selects the
 * K-slice plan (x_amax required): a split-K plan whose workgroups each stay
 * in one K slice and quantize only that slice, the tensor scale taken from
 * the record, workgroup s < splits writing slice s's codes.  The workspace
 * must hold nvfp4_quantize_linear_f32_workspace_bytes(M, N, K) (the largest
 * need of the paths the current options allow), zero-initialised. */
size_t nvfp4_quantize_linear_f32_workspace_bytes(int M, int64_t N, int64_t K);
nvfp4_status nvfp4_quantize_linear_f32(int M, int64_t N, int64_t K, const float* x_f32,
                                       int64_t ldx, const uint32_t* x_amax,
                                       const uint8_t* w_codes, const uint8_t* w_scales,
                                       const float* w_gscale, void* y, int out_dtype,
                                       uint8_t* x_codes, uint8_t* x_scales, float* x_gscale,
                                       void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes nvfp4_linear needs for this shape under the current
 * options: 0 when K is not split, else a fixed 64 KiB region of split-K
 * arrival counters (one per 32-row tile) followed by the binary32 partial
 * sums [splits][M][N_pad].  Because the counters sit at the same place for
 * every shape, one workspace sized for the largest shape serves all. */
size_t nvfp4_linear_workspace_bytes(int M, int64_t N, int64_t K);

/* Zero a workspace before its first use (a fill kernel on `stream`).  The
 * split-K counters reset themselves afterwards, so one initialisation covers
 * any number of later calls, graph replays included.  One workspace must not
 * be used by two calls that can run concurrently. */
nvfp4_status nvfp4_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/* Device self-check of the E2M1 encoder the quantizers use (gfx950's packed
 * FP4 conversion at unit scale) against the rounding rule stated above
 * (nearest, ties to the even code, saturating at 6, sign bit from the input):
 * every finite binary32 pattern is encoded both ways, paired with its
 * negation, both as a lone byte and written into bytes 1, 2 and 3 of a
 * dword whose other bytes must stay.  result: 2 device uint64 (8-byte
 * aligned), overwritten with {mismatches over those four forms, patterns
 * checked}; expect {0, 2^32 - 2^24}.
 * Errors: NVFP4_ERR_INVALID_ARG for a null or misaligned result. */
nvfp4_status nvfp4_selftest_e2m1(unsigned long long* result, void* stream);

/* The decode linear y[m][n] = xgs * wgs * sum_k x[m][k] w[n][k] over the
 * dequantized NVFP4 operands, 1 <= M <= 8, N <= 524288.
 *   x_codes/x_scales canonical activation ([M][K/2], [M][K/16]); x_gscale
 *   and w_gscale device floats; w_codes/w_scales device-tiled weight;
 *   y [M][N] row-major, binary32 or bf16 (round to nearest even);
 *   workspace as sized by nvfp4_linear_workspace_bytes and initialised once
 *   by nvfp4_workspace_init.
 * Accuracy: |y - y_exact| <= 1e-3 * sum_k |x_hat w_hat| per element (plus
 * half a bf16 ulp for bf16 output); the result is bit-identical from run to
 * run (fixed-order split-K reduction). */
nvfp4_status nvfp4_linear(int M, int64_t N, int64_t K, const uint8_t* x_codes,
                          const uint8_t* x_scales, const float* x_gscale, const uint8_t* w_codes,
                          const uint8_t* w_scales, const float* w_gscale, void* y, int out_dtype,
                          void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): exactly
 * nvfp4_quantize_linear (same arguments, same kernels, bit-identical
 * results) without the workspace arguments.  The workspace lives in a
 * library-owned device array of NVFP4_NOALLOC_SCRATCH_BYTES, one per device,
 * held until the process ends; the call allocates nothing.
 *   - Shapes whose nvfp4_quantize_linear_workspace_bytes exceeds
 *     NVFP4_NOALLOC_SCRATCH_BYTES return NVFP4_ERR_WORKSPACE, before any
 *     HIP call.  The default plans of all shapes with N <= 65536, K <= 32768
 *     and M * K <= 204800 (e.g. K <= 25600 at M = 8) fit; larger
 *     activations run the split-K kernel, whose partial sums can exceed it,
 *     and so can forcing many K slices with NVFP4_OPT_SPLIT_K.
 *   - The first call on a device takes the array's device address and
 *     zeroes the array with a fill kernel on `stream`; make that first call
 *     outside stream capture.  Later calls need no clearing (the counters
 *     and the sync record in it return to zero at the end of every call).
 *   - All calls on one device share the one array: calls that can overlap
 *     on one device (different streams without ordering) race and give
 *     wrong results.  Order them on one stream. */
#define NVFP4_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
nvfp4_status nvfp4_quantize_linear_noalloc(int M, int64_t N, int64_t K, const uint16_t* x_bf16,
                                           int64_t ldx, const uint8_t* w_codes,
                                           const uint8_t* w_scales, const float* w_gscale,
                                           void* y, int out_dtype, uint8_t* x_codes,
                                           uint8_t* x_scales, float* x_gscale, void* stream);

/* ------------------------------------------------------------------------
 * ReSET's step-aware decoding temperature (the logits processor of the
 * "ReSET" GitHub README, section "Core components", item 1: the uncertainty
 * of the current reasoning step is estimated online and the temperature set
 * from token- and step-level entropy; t_low and tau0 are the per-model
 * hyper-parameters of the README's "Run benchmarks" command).  The README
 * gives no formula; this library computes, per logits row m:
 *   H_m      = entropy in nats of softmax over the row's V logits
 *              (log sum e^(z - max) - sum e^(z - max) (z - max) / sum e^(z - max),
 *              binary32, reduced in a fixed order: the same on every run;
 *              masked logits (-inf) contribute nothing);
 *   step     = if step_end[m] != 0 (the previous token closed a reasoning
 *              step) the row's running (sum, count) restarts at (0, 0);
 *              then sum += H_m, count += 1, H_step = sum / count;
 *   T_m      = t_low if H_m < tau0, else
 *              min(t_max, t_base * max(1, H_step / tau0));
 *   out[m][v] = logits[m][v] / T_m (one correctly rounded division), if
 *              logits_out is given.
 * Arguments:
 *   logits      [M][ldl] binary32, 16-byte aligned, ldl >= V, ldl % 4 == 0;
 *               every row holds at least one finite logit and no +inf/NaN
 *   M           1..256 rows;  1 <= V <= 2^20 vocabulary entries per row
 *   params      host pointer; every field finite and > 0
 *   step_state  [M][2] device binary32 (running sum, count), zeroed by the
 *               caller when a sequence starts; updated in place
 *   step_end    [M] device int32, or NULL (no step ends)
 *   entropy, temperature  [M] device binary32 outputs
 *   logits_out  [M][ldo] device binary32, 16-byte aligned, ldo >= V,
 *               ldo % 4 == 0, or NULL (not written); may be `logits` itself
 *               (then ldo == ldl), no other overlap
 *   workspace   nvfp4_reset_workspace_bytes(M, V) bytes, 16-byte aligned,
 *               zeroed once by nvfp4_workspace_init; every call leaves its
 *               counters zero again (graph replays need no reset)
 * Two kernels: the row reductions (the last workgroup of a row to finish
 * combines the partials and updates the step state) and the division. */
typedef struct {
  float t_low;   /* temperature of low-entropy tokens (README example 0.1)  */
  float tau0;    /* entropy threshold in nats (README example 0.5505)      */
  float t_base;  /* base temperature of the other tokens                    */
  float t_max;   /* upper bound of the raised temperature                   */
} nvfp4_reset_params;

size_t nvfp4_reset_workspace_bytes(int M, int64_t V);
nvfp4_status nvfp4_reset_temperature(const float* logits, int M, int64_t V, int64_t ldl,
                                     const nvfp4_reset_params* params, float* step_state,
                                     const int32_t* step_end, float* entropy, float* temperature,
                                     float* logits_out, int64_t ldo, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Layer stack: one decode step of an L-layer stack of NVFP4 linears at M
 * rows, captured once into a HIP graph and replayed (the end-to-end figure
 * of the "ReSET" GitHub README, captioned under its introduction, is a
 * 1,500-token Qwen3-32B decode at batch 1 with the step replayed as a
 * graph).  Per layer, in stream order:
 *   RMS norm + quantize (nvfp4_rmsnorm_quantize_act) -> QKV linear
 *   -> quantize the first q_cols columns of its output -> O linear
 *   -> RMS norm + quantize -> gate_up linear (2 * ffn outputs)
 *   -> SiLU * mul + quantize (nvfp4_silu_mul_quantize_act) -> down linear,
 * whose output is the next layer's input.  With gate_up_interleaved set the
 * gate_up linear and SiLU * mul are one call (nvfp4_quantize_linear_silu_mul)
 * and the quantizer of h runs in the down GEMV (nvfp4_quantize_linear_f32
 * with the maxima record), four kernels per layer when every quantizer fits
 * its GEMV's prologue.  Every linear writes bf16.  The
 * stack has no attention, residual or norm weights (out of scope: only the
 * linears and the quantizers between them are modelled).
 */
typedef struct nvfp4_stack nvfp4_stack;

/* One device-tiled weight (as written by nvfp4_quantize_weight). */
typedef struct {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* gscale;
} nvfp4_weight;

typedef struct {
  int M;            /* activation rows, 1..8                                   */
  int layers;       /* 1..4096                                                 */
  int64_t hidden;   /* model width: K of QKV and gate_up, N of O and down      */
  int64_t qkv_n;    /* N of QKV (>= q_cols, multiple of 8)                     */
  int64_t q_cols;   /* leading QKV output columns that feed O (K of O)         */
  int64_t ffn;      /* gate_up has 2 * ffn outputs (gate first); K of down     */
  float eps;        /* RMS norm epsilon, 0 <= eps < 1                          */
  int gate_up_interleaved; /* 1: the gate_up weights come from
                      nvfp4_quantize_weight_gate_up (SiLU * mul fused);
                      0: from nvfp4_quantize_weight (SiLU * mul on its own) */
} nvfp4_stack_config;

/* Create a stack: weights[4 * l + j] is layer l's QKV (j = 0, qkv_n x hidden),
 * O (1, hidden x q_cols), gate_up (2, 2 ffn x hidden), down (3, hidden x ffn);
 * hidden, q_cols and ffn are multiples of 16 up to 32768.
 *   x_in   bf16 [M][hidden], 16-byte aligned: the step's input
 *   y_out  bf16 [M][hidden]: the last layer's down output
 * The caller keeps the weights, x_in and y_out alive and in place while the
 * stack exists (the graph holds their addresses).  `stream` must be a created
 * stream, not the null stream (capture needs one).  Allocates the
 * intermediate activations and a workspace (the only allocations), runs one
 * step eagerly on `stream` (x_in must hold finite values), then captures the
 * step into a graph on `stream`.  On error nothing is left allocated and
 * *out is NULL. */
nvfp4_status nvfp4_stack_create(const nvfp4_stack_config* cfg, const nvfp4_weight* weights,
                                const uint16_t* x_in, uint16_t* y_out, void* stream,
                                nvfp4_stack** out);

/* Replay the captured step `steps` times on `stream` (asynchronous). */
nvfp4_status nvfp4_stack_run(nvfp4_stack* s, int steps, void* stream);

/* The same step launched kernel by kernel, without the graph. */
nvfp4_status nvfp4_stack_run_eager(nvfp4_stack* s, void* stream);

/* Free the stack's buffers and graph (after the work using them is done). */
nvfp4_status nvfp4_stack_destroy(nvfp4_stack* s);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_DECODE_LINEAR_H */
