/*
 * swattn — causal sliding-window attention with RMSNorm on Q and K, forward
 * and backward, for AMD Instinct MI355X (gfx950).  C ABI.
 *
 * The operation is the attention of the single-GPU training step described in
 * the pages on karpathy/autoresearch:
 *   - "Autoresearch 深度教程：AI 自主训练研究指南" (gitee brotherddc/autoresearch),
 *     §5.2.2: each layer attends through a (W, 0) window, W = T/2 for "S"
 *     layers and W = T for "L" layers, pattern "SSSL", last layer always "L";
 *     §5.2.1: the window is handed to FlashAttention-3;
 *     §7.3: `norm(x)` is an RMSNorm over the last axis with no weight.
 *   - okx.com line-by-line review of karpathy/autoresearch: queries and keys
 *     are RMS-normalised right before the attention product (QK-norm).
 *
 * For every batch b and head h, with x[t] the D-vector of position t:
 *   q_hat = q / sqrt(mean(q^2) + eps),  k_hat likewise (unit gain)
 *   key j is visible to query i  iff  0 <= i - j <= W   (W = -1: unbounded)
 *   s_ij  = q_hat_i . k_hat_j / sqrt(D)
 *   o_i   = sum_j softmax_j(s_ij) v_j,   lse_i = ln sum_j exp(s_ij)
 * The softmax scale 1/sqrt(D) is FlashAttention's default; the pages state no
 * other.
 *
 * Layout: q, k, v, o, dout, dq, dk, dv are contiguous bf16 [B, T, H, D]
 * (row-major; element (b, t, h, d) at ((b*T + t)*H + h)*D + d), the layout the
 * tutorial's CausalSelfAttention views its projections in.  lse is fp32
 * [B, H, T].  All tensor and workspace pointers are DEVICE pointers owned by
 * the caller and must be 16-byte aligned (workspaces 256-byte aligned).
 * Outputs are overwritten, never accumulated.  No output may share a byte
 * with an input, another output or the workspace, and the workspace may
 * share none with an input or an output; the library checks this on the
 * byte ranges the sizes imply and rejects a call that breaks it (an output:
 * ATTN_ERR_INVALID_ARG; the workspace: ATTN_ERR_WORKSPACE).  Inputs may
 * overlap each other.
 *
 * Threading / streams: calls are asynchronous on `stream` (a hipStream_t; NULL
 * means the default stream).  The library allocates no device memory, does
 * not synchronise, and keeps no mutable global state apart from the opt-in
 * timing counters below and the device array of attn_fwd_noalloc; concurrent
 * calls on different streams are safe if their buffers are disjoint (for
 * attn_fwd_noalloc, see there).
 *
 * Errors: every argument check runs on the host before any HIP call; a
 * rejected call returns its status and touches nothing.  A failed launch
 * returns ATTN_ERR_HIP.  Faults during execution surface at the caller's next
 * synchronisation, as for any asynchronous HIP work.
 */
#ifndef SWATTN_H
#define SWATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad eps / window, misalignment */
  ATTN_ERR_UNSUPPORTED = 2, /* valid request outside what the kernels implement */
  ATTN_ERR_WORKSPACE = 3,   /* workspace missing, too small, misaligned or overlapping a tensor */
  ATTN_ERR_HIP = 4          /* a HIP launch failed */
};

/* Human-readable name of a status code (static string; never NULL). */
const char* attn_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int attn_version(void);

/*
 * Per-layer windows ("Autoresearch 深度教程" §5.2.2).  Layer l takes the
 * character pattern[l % strlen(pattern)]: 'S' gives seq_len / 2, 'L' gives
 * seq_len (either case accepted); the last layer is always seq_len.  Writes
 * n_layer ints to windows_out (host memory).
 * Returns ATTN_ERR_INVALID_ARG for a NULL/empty pattern, a character other
 * than S/L, n_layer < 1, seq_len < 1 or a NULL windows_out.
 */
int attn_layer_windows(const char* pattern, int n_layer, int seq_len, int* windows_out);

/*
 * Number of visible (query, key) pairs of one (batch, head) slice of length T
 * under `window` (-1 = unbounded), causal only.  Returns -1 for T < 0 or
 * window < -1.  This is the pair count the effective FLOP figures use.
 */
long long attn_visible_pairs(int T, int window);

/*
 * Band tile enumeration used by the kernels.  The rows of a (T x T)
 * query-by-key grid are cut into blocks of `rows` (queries if by_key == 0,
 * keys if by_key == 1) and the other axis into blocks of `cols`.  For every
 * row block r (n = ceil(T / rows) of them) writes, to host arrays of length n:
 *   first[r], last[r] : the first and last column block the kernels visit
 *                       (last < first when none),
 *   n_partial[r]      : how many of the visited blocks need the element mask,
 *   n_empty[r]        : how many of the visited blocks hold no visible pair.
 * Returns ATTN_ERR_INVALID_ARG for T < 1, window < -1, rows/cols < 1 or NULL
 * arrays.
 */
int attn_band_tiles(int T, int window, int rows, int cols, int by_key,
                    int* first, int* last, int* n_partial, int* n_empty);

/* Bytes of device workspace attn_fwd needs: the fp32 [B, H, T] key scales. */
size_t attn_fwd_workspace_bytes(int B, int T, int H, int D);

/*
 * Forward.  q, k, v: bf16 [B, T, H, D] (inputs).  o: bf16 [B, T, H, D]
 * (output).  lse: fp32 [B, H, T] (output; natural log of the sum of exp of the
 * scaled logits of each query row; keep it for attn_bwd).
 * window: W >= 0 keys to the left (W >= T - 1 is full causal), or -1 for full
 * causal.  causal must be 1 (0 returns ATTN_ERR_UNSUPPORTED: the pages never
 * use bidirectional attention).  eps: RMSNorm epsilon, finite and > 0.
 * D must be 64, 128 or 256 (else ATTN_ERR_UNSUPPORTED).  B*T*H*D must stay below
 * 2^31 (else ATTN_ERR_UNSUPPORTED).  B, T or H equal to 0 is an empty problem:
 * returns ATTN_OK and touches nothing (pointers may then be NULL).
 * workspace: device memory of at least attn_fwd_workspace_bytes(B, T, H, D)
 * bytes, 256-byte aligned, contents ignored and clobbered.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             void* workspace, size_t workspace_bytes,
             int B, int T, int H, int D, int window, int causal, float eps,
             void* stream);

/* Bytes of device workspace attn_bwd needs. */
size_t attn_bwd_workspace_bytes(int B, int T, int H, int D);

/*
 * Backward.  Inputs: q, k, v, o (from attn_fwd), lse (from attn_fwd,
 * unchanged), dout = dL/do: bf16 [B, T, H, D] / fp32 [B, H, T].
 * Outputs: dq, dk, dv: bf16 [B, T, H, D], gradients with respect to the
 * PRE-norm q and k and to v.  window, causal, eps, B, T, H, D must equal the
 * forward call's; the same rules and status codes apply.  workspace: at least
 * attn_bwd_workspace_bytes(B, T, H, D) bytes of device memory, 256-byte
 * aligned, clobbered.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, void* dq, void* dk, void* dv,
             void* workspace, size_t workspace_bytes,
             int B, int T, int H, int D, int window, int causal, float eps,
             void* stream);

/*
 * Grouped key/value heads ("Autoresearch 深度教程" §7.3: the attention module
 * has n_kv_head key/value heads, which may be fewer than its n_head query
 * heads; the K and V projections are n_kv_head heads wide).  The pages do not
 * say which query heads share a key/value head; FlashAttention's grouping is
 * used: with G = H / H_kv, query head h reads key/value head h / G.
 *
 * Same contract as attn_fwd / attn_bwd, except that k, v (inputs) and dk, dv
 * (outputs) are bf16 [B, T, H_kv, D]; dk and dv of a shared head are the sums
 * over its G query heads.  H_kv must be >= 1 and divide H (else
 * ATTN_ERR_INVALID_ARG; H_kv < 0 is always invalid, and with H = 0 the call is
 * an empty problem).  H_kv = H is exactly attn_fwd / attn_bwd.  The workspace
 * sizes are those of the *_gqa_workspace_bytes functions.
 */
size_t attn_fwd_gqa_workspace_bytes(int B, int T, int H, int H_kv, int D);
int attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                 void* workspace, size_t workspace_bytes,
                 int B, int T, int H, int H_kv, int D, int window, int causal, float eps,
                 void* stream);
size_t attn_bwd_gqa_workspace_bytes(int B, int T, int H, int H_kv, int D);
int attn_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv,
                 void* workspace, size_t workspace_bytes,
                 int B, int T, int H, int H_kv, int D, int window, int causal, float eps,
                 void* stream);

/*
 * Rotary position embedding fused into the QK-norm prologue ("Autoresearch
 * 深度教程" §7.4 defines the rotation and its bf16 cos/sin tables; §7.3's
 * attention module rotates q and k and then normalises them).  q and k are the
 * projections BEFORE the rotation.  The operation is attn_fwd_gqa applied to
 * rope(q) and rope(k), where for position t and channel i < D/2
 *   rope(x)[i]       = x[i] cos[t, i] + x[i + D/2] sin[t, i]
 *   rope(x)[i + D/2] = x[i + D/2] cos[t, i] - x[i] sin[t, i]
 * (the same tables for q and k), and attn_bwd_rope returns dq and dk with
 * respect to the q and k before the rotation.
 * rope_cos, rope_sin: bf16 [T, D/2] device tables, row t for position t (for
 * example the first T rows of a model's precomputed [1, T', 1, D/2] buffers),
 * 16-byte aligned, read only; they must not alias an output.  All other rules
 * are those of the *_gqa entry points; the workspace adds a bf16 copy of the
 * rotated keys: *_rope_workspace_bytes.
 */
size_t attn_fwd_rope_workspace_bytes(int B, int T, int H, int H_kv, int D);
int attn_fwd_rope(const void* q, const void* k, const void* v,
                  const void* rope_cos, const void* rope_sin, void* o, float* lse,
                  void* workspace, size_t workspace_bytes,
                  int B, int T, int H, int H_kv, int D, int window, int causal, float eps,
                  void* stream);
size_t attn_bwd_rope_workspace_bytes(int B, int T, int H, int H_kv, int D);
int attn_bwd_rope(const void* q, const void* k, const void* v,
                  const void* rope_cos, const void* rope_sin,
                  const void* o, const float* lse, const void* dout,
                  void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                  int B, int T, int H, int H_kv, int D, int window, int causal, float eps,
                  void* stream);

/*
 * Value-embedding gate fused into the V load ("Autoresearch 深度教程" §5.2.3:
 * a layer with a value embedding ve mixes it into v through a gate computed
 * per token and key/value head from the first 32 channels of the block input
 * x by a bias-free linear map W_g):
 *   gate[b, t, h] = 2 sigmoid(sum_{c < 32} gate_w[h, c] x[b, t, c]),
 *   attention uses v + gate * ve in place of v.
 * ve: bf16 [B, T, H_kv, D].  xg: bf16 gate input, token (b, t) at
 * xg + (b T + t) xg_stride elements, channels 0..31 read (a [B, T, C] block
 * input with xg_stride = C works as is); xg_stride >= 32 and a multiple of 8.
 * gate_w: fp32 [H_kv, 32].  rope_cos / rope_sin: as in attn_fwd_rope, or both
 * NULL for no rotation.  H_kv above 16 returns ATTN_ERR_UNSUPPORTED.
 * attn_bwd_ve also writes dve (bf16 [B, T, H_kv, D]), dxg (bf16 [B, T, 32]:
 * the gradient of x's first 32 channels; the other channels get none) and
 * dgate_w (fp32 [H_kv, 32], summed over all tokens in a fixed order, so
 * deterministic); dv is the gradient of v.  Every output must be 16-byte
 * aligned and alias no input or other output.  Other rules as for the
 * *_gqa entry points; workspace sizes: *_ve_workspace_bytes (those of the
 * *_rope entry points plus a bf16 [B, T, H_kv, D] copy of the gated values
 * and the fp32 [B, H_kv, T] gate, and for the backward the gate's gradients).
 */
size_t attn_fwd_ve_workspace_bytes(int B, int T, int H, int H_kv, int D);
int attn_fwd_ve(const void* q, const void* k, const void* v, const void* ve,
                const void* xg, int xg_stride, const float* gate_w,
                const void* rope_cos, const void* rope_sin, void* o, float* lse,
                void* workspace, size_t workspace_bytes,
                int B, int T, int H, int H_kv, int D, int window, int causal, float eps,
                void* stream);
size_t attn_bwd_ve_workspace_bytes(int B, int T, int H, int H_kv, int D);
int attn_bwd_ve(const void* q, const void* k, const void* v, const void* ve,
                const void* xg, int xg_stride, const float* gate_w,
                const void* rope_cos, const void* rope_sin,
                const void* o, const float* lse, const void* dout,
                void* dq, void* dk, void* dv, void* dve, void* dxg, float* dgate_w,
                void* workspace, size_t workspace_bytes,
                int B, int T, int H, int H_kv, int D, int window, int causal, float eps,
                void* stream);

/*
 * Backward passes that reuse the forward's key pre-pass.  Both passes start
 * with the same per-key work (the QK-RMSNorm scale of every key row of the
 * "Autoresearch 深度教程" §7.3 norm, and with the §7.4 rotary embedding or the
 * §5.2.3 value-embedding gate the rotated keys, the gated values and the
 * gate).  The forward keeps it in its workspace; these entry points read it
 * there instead of computing it again, which saves one pass over K (and over
 * V and ve with the gate).
 * fwd_workspace: the workspace of the attn_fwd / attn_fwd_gqa, attn_fwd_rope
 * or attn_fwd_ve call (the matching variant, same problem, tables, gate
 * inputs and eps) that produced o and lse, unchanged since that call;
 * fwd_workspace_bytes at least that variant's *_workspace_bytes, 256-byte
 * aligned, read only, and distinct from workspace and every output.
 * workspace: this call's own, sized as for the corresponding backward.
 * Results are bit-identical to the corresponding backward; every other
 * argument, rule and status code is the same.  A NULL or too small
 * fwd_workspace returns ATTN_ERR_WORKSPACE.
 */
int attn_bwd_gqa_reuse(const void* q, const void* k, const void* v, const void* o,
                       const float* lse, const void* dout, void* dq, void* dk, void* dv,
                       const void* fwd_workspace, size_t fwd_workspace_bytes,
                       void* workspace, size_t workspace_bytes,
                       int B, int T, int H, int H_kv, int D, int window, int causal, float eps,
                       void* stream);
int attn_bwd_rope_reuse(const void* q, const void* k, const void* v,
                        const void* rope_cos, const void* rope_sin,
                        const void* o, const float* lse, const void* dout,
                        void* dq, void* dk, void* dv,
                        const void* fwd_workspace, size_t fwd_workspace_bytes,
                        void* workspace, size_t workspace_bytes,
                        int B, int T, int H, int H_kv, int D, int window, int causal, float eps,
                        void* stream);
int attn_bwd_ve_reuse(const void* q, const void* k, const void* v, const void* ve,
                      const void* xg, int xg_stride, const float* gate_w,
                      const void* rope_cos, const void* rope_sin,
                      const void* o, const float* lse, const void* dout,
                      void* dq, void* dk, void* dv, void* dve, void* dxg, float* dgate_w,
                      const void* fwd_workspace, size_t fwd_workspace_bytes,
                      void* workspace, size_t workspace_bytes,
                      int B, int T, int H, int H_kv, int D, int window, int causal, float eps,
                      void* stream);

/*
 * Forward that allocates nothing, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops and harnesses
 * that forbid allocation.  Same operation, arguments, rules and status codes
 * as attn_fwd, without the workspace: the key scales live in a device array
 * of the library (attn_fwd_noalloc_max_bytes() = 8 MiB, so B*H*T <= 2^21),
 * which each GPU holds from the library's first use on it until the process
 * ends.  A problem whose attn_fwd_workspace_bytes exceed that size returns
 * ATTN_ERR_WORKSPACE and touches nothing.  Every call on one GPU shares the
 * array: calls that overlap in time on one GPU (other streams, other host
 * threads) race on it.  A backward may not reuse it as a forward workspace
 * (the next call overwrites it); run attn_bwd.  Results equal attn_fwd's bit
 * for bit.
 */
size_t attn_fwd_noalloc_max_bytes(void);
int attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int T, int H, int D, int window, int causal, float eps,
                     void* stream);

/*
 * Opt-in per-kernel timing, a measurement aid (not part of the operation).
 * While enabled, every kernel launch of attn_fwd / attn_bwd is bracketed by
 * two HIP events recorded on the launch stream.  Kernel ids: 0 fwd_prep
 * (the key pre-pass launched by the forward: key scales, and the rotated keys
 * or gated values when used), 1 attn_fwd (forward attention),
 * 2 bwd_kscale (the same pre-pass launched by the backward), 3 bwd_dkdv (dK and dV),
 * 4 bwd_dq (dQ, with q_hat, Delta and lse log2(e) for bwd_dkdv),
 * 5 bwd_gate (the value-embedding gate's dx and dW_g, attn_bwd_ve only).
 *   attn_profile_enable(on): clears the totals and starts (on != 0) or stops
 *     recording; returns ATTN_ERR_HIP if waiting on earlier events failed.
 *   attn_profile_enable_mask(mask): the same, recording only the kernels
 *     whose bit (1 << id) is set in mask (0 stops).  Each recorded launch
 *     costs its stream a few microseconds for the two events, so a caller
 *     that times whole steps records as few kernels as it needs.
 *   attn_profile_read(kernel, total_ms, launches): waits for the recorded
 *     events and returns the summed milliseconds and launch count of that
 *     kernel since the last enable; ATTN_ERR_INVALID_ARG for a bad id or NULL.
 *   attn_kernel_name(kernel): the kernel's name ("unknown" if out of range).
 * This is the library's only mutable global state; it is mutex-protected.
 */
int attn_profile_enable(int on);
int attn_profile_enable_mask(unsigned mask);
int attn_profile_read(int kernel, double* total_ms, long long* launches);
const char* attn_kernel_name(int kernel);

/*
 * Device facts a roofline needs, another measurement aid: the number of
 * compute units of HIP device `device` and its peak shader clock in kHz (HIP's
 * hipDeviceAttributeClockRate).  A bf16 dense MFMA peak follows as
 * compute_units x 4096 FLOP per clock x clock on gfx950.  Returns
 * ATTN_ERR_INVALID_ARG for a NULL output or a negative device, ATTN_ERR_HIP if
 * the runtime cannot answer (no such device).  Initialises the HIP runtime.
 */
int attn_device_info(int device, int* compute_units, int* max_clock_khz);

#ifdef __cplusplus
}
#endif

#endif /* SWATTN_H */
