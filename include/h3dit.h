/*
 * h3dit.h -- C ABI of the MI355X (gfx950) MiniMax-H3 DiT block forward.
 *
 * What is computed (page titles and sections):
 *   One DiT block, run 50 times per denoising forward, over one packed
 *   sequence [text | conditions | audio | video]: full self-attention, no
 *   cross-attention, modality entering only through a per-row AdaLN tag that
 *   reads a precomputed per-timestep modulation table
 *   ("minimax-h3-mlx README", sections "Architecture" and "AdaLN precompute").
 *   Per block and row r with tag m:
 *     h   = LN(x) * (1 + scale1[m]) + shift1[m]
 *     q,k,v = split_per_head(h W_qkv^T + b_qkv)        (rows interleaved per head)
 *     q,k = RoPE3D(RMSNorm(q) * g_q), RoPE3D(RMSNorm(k) * g_k)
 *     o   = softmax(q k^T / sqrt(d)) v                  (all rows, no mask)
 *     x  += gate1[m] * (o W_out^T + b_out)
 *     h2  = LN(x) * (1 + scale2[m]) + shift2[m]
 *     x  += gate2[m] * (swiglu(h2 W_fc1^T + b_fc1) W_fc2^T + b_fc2)
 *   ("minimax-h3-mlx README", "Validation" for the QKV interleave and the
 *   fused [gate; value] fc1; "AdaLN: measure, do not reason" for the six
 *   modulation tensors; "H3-metal" digest, "Checkpoint layout and media
 *   pipeline" for QK normalisation before RoPE.)
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers, 16-byte aligned, owned by the
 *     caller.  The library allocates no device memory and keeps no pointer
 *     after a call returns.  bf16 values are passed as uint16_t bit patterns.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = default stream) and
 *     the call returns before it completes.  Calls that share a workspace or
 *     an output buffer must be ordered by the caller (same stream).
 *   - Every argument is checked on the host before anything is enqueued.  On
 *     an error nothing is enqueued, a negative h3_status is returned and
 *     h3_last_error() (thread-local) describes it.  There is no fallback to
 *     another implementation: unsupported shapes are errors.
 *   - Matrix layouts are row-major.  Linear weights use the PyTorch layout
 *     W[out][in].  n_pad = h3_padded_rows(n_rows) (a multiple of 256).
 *   - Modality tags must lie in [0, n_tags).  They are not checked unless
 *     H3_CHECK=1 is set in the environment: then every call that reads tags
 *     first scans them on the device (one small kernel counting into a
 *     4-byte counter in the library's static device memory, and a wait for
 *     the stream, so not under stream capture; check-mode calls that overlap
 *     on one device share the counter) and returns H3_ERR_INVALID_ARG, with
 *     nothing else enqueued, if any lies outside that range.
 *   - H3_UNFUSED=1 in the environment (a debugging switch, read at every
 *     call): the block forwards with bf16 weights run each GEMM with a plain
 *     fp32 store of acc + bias and its epilogue (QK-RMSNorm + RoPE + q scale +
 *     head-major scatter, SwiGLU, gated residual) as a separate elementwise
 *     kernel, to compare the fused epilogues against (the pages keep unfused
 *     two-kernel versions of their fused kernels switchable in the same way:
 *     H3-metal digest, "Exact DiT fusions").  h3_workspace_size then adds one
 *     fp32 buffer of n_pad x max(3 * heads * head_dim, 2 * ffn, hidden), so
 *     the switch must be the same when a workspace is sized and when it is
 *     used.  Other weight formats and the step entry points ignore it.
 *
 * Supported shapes: hidden % 256 == 0 and hidden <= 8192; head_dim in
 * {96, 128}; ffn % 128 == 0 and (ffn + 256) * hidden * 2 < 2^32; rope_split
 * entries even and summing to head_dim; 1 <= n_tags <= 8;
 * 1 <= n_rows <= 2^24; with INT8 weights also heads * head_dim % 128 == 0.
 */
#ifndef H3DIT_H
#define H3DIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define H3DIT_API __attribute__((visibility("default")))

typedef enum h3_status {
  H3_OK = 0,
  H3_ERR_INVALID_ARG = -1, /* null / misaligned pointer, bad size or field */
  H3_ERR_UNSUPPORTED = -2, /* well-formed but outside the supported shapes */
  H3_ERR_WORKSPACE = -3,   /* workspace smaller than h3_workspace_size()  */
  H3_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed   */
  H3_ERR_NO_DEVICE = -5    /* no usable GPU                                */
} h3_status;

typedef enum h3_wfmt {
  H3_W_BF16 = 0,     /* weights bf16 [out][in]                                    */
  H3_W_INT8_G32 = 1, /* weights int8 [out][in] + bf16 scales [out][in/32]:
                        W = bf16(q * s), one scale per 32 consecutive K elements  */
  H3_W_W8A8 = 2      /* group-scaled W8A8 (mlx-h3 README, "Generate": the 200
                        trunk linears as group-scaled W8A8, groups of 64, 256,
                        448 or 896 along K): weights int8 [out][in] + bf16
                        scales [in/G][out] (group-major), G = dims->w8a8_group;
                        each linear's bf16 input is quantized per row and group
                        (amax = max|a| over the group, q = clamp(rint(a *
                        (127 / amax)), +-127), scale amax / 127, in float32) and
                        y = b + sum_g s_a[r][g] s_w[g][c] sum_{k in g} q_a q_w,
                        each group's sum in int32 on the int8 matrix cores.
                        With dims->w8a8_row_fc2 = 1, FC2 alone takes one scale
                        per activation row and per weight output row (scales
                        [out]; H3-metal digest, "4. Choose a speed/quality
                        preset": the per-row FC2 option).                      */
} h3_wfmt;

typedef struct h3_dims {
  int32_t hidden;        /* D: 5376 for H3                                     */
  int32_t heads;         /* H: 56                                              */
  int32_t head_dim;      /* d: 128 (96 or 128 supported)                       */
  int32_t ffn;           /* F: 14336 (SwiGLU width)                            */
  int32_t n_tags;        /* T: modality groups in the table (3)                */
  int32_t rope_split[3]; /* head_dim channels given to the t, h, w axes        */
  float rope_theta;      /* rotary base (10000)                                */
  float ln_eps;          /* AdaLN layer-norm epsilon (1e-6)                    */
  float qk_eps;          /* QK RMSNorm epsilon (1e-6)                          */
  int32_t wfmt;          /* h3_wfmt of the four linear layers                  */
  int32_t w8a8_group;    /* H3_W_W8A8: K elements per scale group, one of 64,
                            256, 448, 896, dividing hidden, heads*head_dim and
                            ffn (ffn not needed with w8a8_row_fc2); else ignored */
  int32_t w8a8_row_fc2;  /* H3_W_W8A8: 1 = FC2 with per-row scales, 0 = grouped */
} h3_dims;

/* Device pointers of one block's weights.  w_qkv [3*H*d][D] rows interleaved
 * per head ([h0: q,k,v][h1: q,k,v]...), w_out [D][H*d], w_fc1 [2F][D] stacked
 * [gate; value], w_fc2 [D][F].  s_* are the INT8 scales (ignored for bf16).
 * Biases b_* (bf16 [out]) and the QK-norm gains q_norm / k_norm (bf16 [d])
 * may be NULL, meaning 0 and 1. */
typedef struct h3_block_weights {
  const void *w_qkv, *w_out, *w_fc1, *w_fc2;
  const uint16_t *s_qkv, *s_out, *s_fc1, *s_fc2;
  const uint16_t *b_qkv, *b_out, *b_fc1, *b_fc2;
  const uint16_t *q_norm, *k_norm;
} h3_block_weights;

/* ------------------------------------------------------------------------ */
/* Whole-path entry points                                                   */
/* ------------------------------------------------------------------------ */

/* Rows rounded up to the kernels' row tile (256).  Pure. */
H3DIT_API int64_t h3_padded_rows(int64_t n_rows);

/* Bytes of scratch a forward over n_rows needs.  Pure: touches no device.
 * Returns 0 if dims or n_rows are invalid (h3_last_error() says why).
 * With INT8 weights (H3_W_INT8_G32) this includes one linear's dequantised
 * bf16 weights (2 * 2 * ffn * hidden bytes, FC1's, the largest: 308 MB at H3
 * width): the forward then forms each linear's bf16 weights there once and
 * runs the bf16 GEMM on them.  A workspace that lacks only that buffer is
 * accepted too, and runs the INT8 GEMMs on the kernel that dequantises the
 * weights in LDS per row tile (same values, the weights round to
 * RNE_bf16(q * s) either way). */
H3DIT_API size_t h3_workspace_size(const h3_dims* dims, int64_t n_rows);

/* One DiT block in place.
 *   x          fp32 [n_rows][D]   residual stream, read and overwritten
 *   tag        int32 [n_rows]     modality tag of each packed row
 *   positions  fp32 [n_rows][3]   (t, h, w) rotary coordinates of each row
 *   mod_table  bf16 [T][6][D]     this block's modulation vectors, in the
 *                                 order shift1, scale1, gate1, shift2,
 *                                 scale2, gate2 (minimax-h3-mlx README,
 *                                 "AdaLN precompute": 18*D per timestep)
 *   weights    host pointer to one h3_block_weights (device pointers inside)
 *   workspace  device scratch of at least h3_workspace_size() bytes       */
H3DIT_API h3_status h3_dit_block_forward(const h3_dims* dims, float* x, const int32_t* tag,
                                         const float* positions, const uint16_t* mod_table,
                                         const h3_block_weights* weights, int64_t n_rows,
                                         void* workspace, size_t workspace_bytes, void* stream);

/* One denoising forward: blocks 0..n_blocks-1 in order, in place on x.
 *   mod_table  bf16 [n_blocks][T][6][D]
 *   weights    host array of n_blocks h3_block_weights
 * The rotary table is built once and shared by all blocks. */
H3DIT_API h3_status h3_dit_forward(const h3_dims* dims, float* x_packed, const int32_t* tag,
                                   const float* positions, const uint16_t* mod_table,
                                   const h3_block_weights* weights, int32_t n_blocks,
                                   int64_t n_rows, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* Size of the library's own scratch array on each GPU (128 MiB), the largest
 * workspace h3_dit_forward_noalloc can use. */
#define H3_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/* h3_dit_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same blocks, kernels and results, with the workspace taken from the
 * library's static scratch array (H3_NOALLOC_SCRATCH_BYTES per GPU, held from
 * the library's first use of that GPU until the process ends) instead of a
 * caller buffer.  Calls nothing that allocates.  Fails with H3_ERR_WORKSPACE
 * when h3_workspace_size(dims, n_rows) exceeds the array: at H3 width that is
 * above 1,792 rows with bf16 or INT8 weights and above 1,536 rows with W8A8.
 * Every call on one GPU uses the same array (nothing in it has to start at
 * zero, and the last call's contents stay there): calls that overlap on one
 * GPU, on any streams, race and give undefined results. */
H3DIT_API h3_status h3_dit_forward_noalloc(const h3_dims* dims, float* x_packed, const int32_t* tag,
                                           const float* positions, const uint16_t* mod_table,
                                           const h3_block_weights* weights, int32_t n_blocks,
                                           int64_t n_rows, void* stream);

/* h3_dit_forward with block-sparse attention in every block (see
 * h3_attention_sparse): block b reads its selection from the CSR offsets
 * tile_off + b * (heads*nq + 1), which index the one array tile_idx.  Each
 * block's offsets follow the rules of h3_attention_sparse except that they
 * start where that block's lists start in tile_idx; every offset must lie in
 * [0, len(tile_idx)]. */
H3DIT_API h3_status h3_dit_forward_sparse(const h3_dims* dims, float* x_packed, const int32_t* tag,
                                          const float* positions, const uint16_t* mod_table,
                                          const h3_block_weights* weights, int32_t n_blocks,
                                          int64_t n_rows, int32_t tile, const int32_t* tile_off,
                                          const int32_t* tile_idx, void* workspace,
                                          size_t workspace_bytes, void* stream);

/* Message of the last error on this thread ("" if none).  Never NULL. */
H3DIT_API const char* h3_last_error(void);


/* W8A8 activation buffer of width K and scale group G (G = K: one scale per
 * row): int8 codes [n_rows][K], then at byte offset roundup(n_rows * K, 256)
 * fp32 scales [K/G][n_pad] (group-major, n_pad = h3_padded_rows(n_rows), the
 * rows past n_rows holding 0).  Bytes it needs (pure; 0 for invalid sizes). */
H3DIT_API size_t h3_quantized_bytes(int64_t n_rows, int32_t width, int32_t group);

/* Symmetric int8 quantization (the H3_W_W8A8 rule) of in bf16 [n_rows][width]
 * per row and group of `group` consecutive elements (64, 256, 448, 896, or
 * group == width for one scale per row) into the activation buffer out.
 * width % 8 == 0, width % group == 0, width <= 16384. */
H3DIT_API h3_status h3_quantize_groups(const uint16_t* in, int64_t n_rows, int32_t width,
                                       int32_t group, void* out, void* stream);

/* ------------------------------------------------------------------------ */
/* Around the block stack: inputs -> packed stream -> velocity               */
/* ------------------------------------------------------------------------ */
/* The packed stream's rows come from four inputs, in the order
 * [text | conditions | audio | video] (minimax-h3-mlx README, "Architecture"):
 *   text rows   = text_hidden W_text^T + b_text     (the text encoder's
 *                 unnormalised hidden state, width 5120, into the DiT's
 *                 condition projection: minimax-h3-mlx README, "Encoder
 *                 truncation"); bf16 weights, fp32 accumulation.
 *   cond rows   = cond_patch W_video^T + b_video     (keyframes are video
 *                 latents; only two patch projections exist)
 *   audio rows  = audio_patch W_audio^T + b_audio
 *   video rows  = video_patch W_video^T + b_video
 * The patch projections keep fp32 weights, inputs and accumulation (H3-metal
 * digest, "Specialized projection kernels": 96 -> 5376 video, 32 -> 5376
 * audio, fp32; minimax-h3-mlx README, "Published quants": these tensors ship
 * in fp32).  After the blocks, the audio and the video slice each take a final
 * AdaLN, h = LN(x) * (1 + scale_m) + shift_m, and their output head,
 * vel = h W_head^T + b_head, with bf16 head weights (converted once from the
 * released fp32 ones) on bf16 h, fp32 accumulation (H3-metal digest,
 * "Exact DiT fusions" and "Specialized projection kernels").  Text and
 * condition rows get no velocity. */
typedef struct h3_io_dims {
  int32_t text_dim;    /* text hidden-state width (5120); a multiple of 64       */
  int32_t video_patch; /* video latent patch width (96 = 24 ch x 1x2x2); 32, 64, 96 or 128 */
  int32_t audio_patch; /* audio latent patch width (32); 32, 64, 96 or 128       */
} h3_io_dims;

/* Row counts of the four segments; the stream has text+cond+audio+video rows. */
typedef struct h3_segments {
  int64_t text, cond, audio, video;
} h3_segments;

/* Device pointers.  Weights in PyTorch layout W[out][in]; biases nullable (0).
 * Pointers of a segment with no rows may be NULL. */
typedef struct h3_io_weights {
  const uint16_t* w_text;       /* bf16 [D][text_dim]     condition projection    */
  const uint16_t* b_text;       /* bf16 [D]                                       */
  const float* w_video;         /* fp32 [D][video_patch]  video + condition rows  */
  const float* b_video;         /* fp32 [D]                                       */
  const float* w_audio;         /* fp32 [D][audio_patch]                          */
  const float* b_audio;         /* fp32 [D]                                       */
  const uint16_t* w_head_audio; /* bf16 [audio_patch][D]  audio output head       */
  const uint16_t* b_head_audio; /* bf16 [audio_patch]                             */
  const uint16_t* w_head_video; /* bf16 [video_patch][D]  video output head       */
  const uint16_t* b_head_video; /* bf16 [video_patch]                             */
} h3_io_weights;

/* Bytes of scratch h3_final_heads needs (max(audio, video) rows of bf16 h).
 * Pure.  Returns 0 on invalid dims or segments. */
H3DIT_API size_t h3_heads_workspace_size(const h3_dims* dims, const h3_segments* segments);

/* Writes every row of x_packed fp32 [N][D] from the inputs:
 *   text bf16 [text][text_dim]; cond fp32 [cond][video_patch];
 *   audio fp32 [audio][audio_patch]; video fp32 [video][video_patch]. */
H3DIT_API h3_status h3_embed_inputs(const h3_dims* dims, const h3_io_dims* io_dims,
                                    const h3_io_weights* io_weights, const h3_segments* segments,
                                    const uint16_t* text, const float* cond, const float* audio,
                                    const float* video, float* x_packed, void* stream);

/* Velocities from the stream x_packed fp32 [N][D] (read only):
 *   final_table bf16 [2][2][D]: (audio, video) x (shift, scale) of the final
 *               AdaLN for this timestep (precomputed like mod_table)
 *   vel_audio   fp32 [audio][audio_patch];  vel_video fp32 [video][video_patch]
 *   workspace   at least h3_heads_workspace_size() bytes */
H3DIT_API h3_status h3_final_heads(const h3_dims* dims, const h3_io_dims* io_dims,
                                   const h3_io_weights* io_weights, const h3_segments* segments,
                                   const float* x_packed, const uint16_t* final_table,
                                   float* vel_audio, float* vel_video, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* One velocity forward: h3_embed_inputs into x_packed (which the caller
 * provides and which ends holding the last block's output), n_blocks blocks
 * as h3_dit_forward (n_blocks may be 0: then tag, positions, mod_table and
 * weights may be NULL and the workspace needs only h3_heads_workspace_size()
 * bytes, else h3_workspace_size(dims, N)), then h3_final_heads. */
H3DIT_API h3_status h3_velocity_forward(const h3_dims* dims, const h3_io_dims* io_dims,
                                        const h3_io_weights* io_weights,
                                        const h3_segments* segments, const uint16_t* text,
                                        const float* cond, const float* audio, const float* video,
                                        const int32_t* tag, const float* positions,
                                        const uint16_t* mod_table,
                                        const h3_block_weights* weights, int32_t n_blocks,
                                        const uint16_t* final_table, float* x_packed,
                                        float* vel_audio, float* vel_video, void* workspace,
                                        size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Step entry points: each runs one step of the block on caller buffers.     */
/* They are the kernels h3_dit_block_forward launches, exposed for parity   */
/* tests and per-step timing.  With dims->wfmt == H3_W_W8A8 the bf16         */
/* inputs of the four linears (h, h2, o, a) are W8A8 activation buffers     */
/* instead (h3_quantized_bytes with the linear's group: w8a8_group, or K    */
/* for FC2 with w8a8_row_fc2), made by h3_quantize_groups from the bf16     */
/* tensors (h3_adaln_modulate always writes bf16).                          */
/* ------------------------------------------------------------------------ */

/* Rotary table: cs fp32 [n_pad][d/2][2] = (cos, sin) of the angle of every
 * channel pair; pair j of axis a (width d_a) turns by
 * positions[r][a] * theta^(-2j/d_a).  Rows >= n_rows get angle 0.
 * ("minimax-h3-mlx README", "Architecture": 3D MM-RoPE.) */
H3DIT_API h3_status h3_rope_table(const h3_dims* dims, const float* positions, int64_t n_rows,
                                  float* cs, void* stream);

/* AdaLN norm-modulate: h bf16 [n_rows][D] = LN(x) * (1 + scale) + shift with
 * (shift, scale) = mod_table[tag][3*which + 0 / 1]; which = 0 before
 * attention, 1 before the MLP.  LN: no affine, biased variance, ln_eps. */
H3DIT_API h3_status h3_adaln_modulate(const h3_dims* dims, const float* x, const int32_t* tag,
                                      const uint16_t* mod_table, int32_t which, int64_t n_rows,
                                      uint16_t* h, void* stream);

/* Fused QKV projection + per-head RMSNorm + RoPE + head-major scatter.
 *   h   bf16 [n_rows][D]
 *   cs  the rotary table from h3_rope_table
 *   q   bf16 [H][n_pad][d], pre-multiplied by log2(e)/sqrt(d)
 *   k   bf16 [H][n_pad][d]
 *   vt  bf16 [H][d][n_pad]  (v transposed: keys contiguous)
 * Rows n_rows..n_pad-1 of q, k and vt are written as zeros. */
H3DIT_API h3_status h3_qkv_rope(const h3_dims* dims, const uint16_t* h,
                                const h3_block_weights* weights, const float* cs, int64_t n_rows,
                                uint16_t* q, uint16_t* k, uint16_t* vt, void* stream);

/* Full attention over all n_rows keys (no mask): o bf16 [n_rows][H*d], head
 * h in columns [h*d, (h+1)*d).  q, k, vt as written by h3_qkv_rope. */
H3DIT_API h3_status h3_attention(const h3_dims* dims, const uint16_t* q, const uint16_t* k,
                                 const uint16_t* vt, int64_t n_rows, uint16_t* o, void* stream);

/* Block-sparse attention: query tile i (rows [i*tile, (i+1)*tile)) of head h
 * attends only to the keys of the key tiles j (rows [j*tile, (j+1)*tile), the
 * last tile ragged) listed in tile_idx[tile_off[h*nq + i] .. tile_off[h*nq + i + 1]),
 * nq = ceil(n_rows / tile), tile 64 or 128 (FastH3 OmniRef (Ref2VA) on Apple
 * Silicon MLX, "Opt-in M5 attention backend": selected 64/128 tiles, only
 * their valid rows visited).  tile_off int32 [heads*nq + 1] and tile_idx int32
 * are device arrays (4-byte aligned); tile_off is non-decreasing, starts at 0
 * and its last entry is the length of tile_idx.  The library does not read
 * them on the host: an offset outside [0, len(tile_idx)] makes the kernel read
 * outside tile_idx.  Lists need not be sorted and must hold no duplicates (a
 * repeated tile counts its keys twice); indices outside [0, nq) are clamped,
 * lists longer than nq are cut at nq entries, an empty list gives zero rows.
 * q, k, vt, o as for h3_attention. */
H3DIT_API h3_status h3_attention_sparse(const h3_dims* dims, const uint16_t* q, const uint16_t* k,
                                        const uint16_t* vt, int64_t n_rows, int32_t tile,
                                        const int32_t* tile_off, const int32_t* tile_idx,
                                        uint16_t* o, void* stream);

/* x fp32 [n_rows][D] += gate1[tag] * (o W_out^T + b_out);  o bf16 [n_rows][H*d]. */
H3DIT_API h3_status h3_out_proj_residual(const h3_dims* dims, const uint16_t* o,
                                         const h3_block_weights* weights,
                                         const uint16_t* mod_table, const int32_t* tag,
                                         int64_t n_rows, float* x, void* stream);

/* a bf16 [n_rows][F] = silu(z[:, :F]) * z[:, F:],  z = h2 W_fc1^T + b_fc1. */
H3DIT_API h3_status h3_mlp_fc1_swiglu(const h3_dims* dims, const uint16_t* h2,
                                      const h3_block_weights* weights, int64_t n_rows,
                                      uint16_t* a, void* stream);

/* x fp32 [n_rows][D] += gate2[tag] * (a W_fc2^T + b_fc2);  a bf16 [n_rows][F]. */
H3DIT_API h3_status h3_mlp_fc2_residual(const h3_dims* dims, const uint16_t* a,
                                        const h3_block_weights* weights,
                                        const uint16_t* mod_table, const int32_t* tag,
                                        int64_t n_rows, float* x, void* stream);

/* ------------------------------------------------------------------------ */
/* Denoising loop: rectified-flow Euler, one velocity forward per pass       */
/* ------------------------------------------------------------------------ */
/* Sigmas of one modality's schedule, host double [n_steps + 1]: base grid
 * b_i = 1 - i/n_steps (i < n_steps), exponentially shifted to
 * shift*b / (1 + (shift - 1)*b), then the terminal 0 (minimax-h3-mlx README,
 * "Layout": rectified-flow Euler with exponential sigma shift; "AdaLN
 * precompute": video shift 12.0, audio 3.0, whose 40-pass schedules meet in 77
 * distinct timesteps; H3-metal digest, "Sampler and DiT controls": terminal
 * zero after the last pass).  Pure host function. */
H3DIT_API h3_status h3_sigma_schedule(int32_t n_steps, double shift, double* sigmas);

/* n_steps Euler passes on the GPU.  A fresh pass i runs the velocity forward
 * (h3_velocity_forward with the current latents, the blocks' tables
 * mod_tables + i*n_blocks*T*6*D and the final table final_tables + i*2*2*D);
 * then every pass steps, per modality,  z += (sigma[i+1] - sigma[i]) * v.
 * Whole-velocity reuse (H3-metal digest, "4. Choose a speed/quality preset":
 * at 20 passes, reuse 1, 2, 3 make 20, 11, 8 fresh evaluations; "Sampler and
 * DiT controls": the skipped video and audio velocities are extrapolated on
 * their independent schedules): pass i is fresh when i % reuse == 0 or it is
 * the last pass.  A skipped pass i steps each modality m along
 *   v1 + (sigma_m[i] - sigma_m[j1]) / (sigma_m[j1] - sigma_m[j0]) * (v1 - v0),
 * the straight line in that modality's sigma through its last two fresh
 * velocities v0 (pass j0) and v1 (pass j1 > j0); while only one fresh velocity
 * exists (right after pass 0) it steps along that one.  reuse >= 1 (1: every
 * pass fresh).
 *   audio fp32 [audio][audio_patch], video fp32 [video][video_patch]: the
 *         latents, updated in place (text and condition inputs stay fixed)
 *   mod_tables bf16 [n_steps][n_blocks][T][6][D]; final_tables bf16
 *         [n_steps][2][2][D] (each step's tables from its own per-modality
 *         timesteps, precomputed as in "AdaLN precompute")
 *   sigmas_audio, sigmas_video: host double [n_steps + 1] (h3_sigma_schedule)
 *   x_packed fp32 [N][D]: scratch for the stream; workspace at least
 *         h3_denoise_workspace_size() bytes: the block workspace, then the
 *         last two fresh velocities of each modality.  n_blocks >= 1. */
/* Workspace bytes of h3_denoise: h3_workspace_size(dims, N) plus two fp32
 * velocity slots per modality ([audio][audio_patch] and [video][video_patch]),
 * each rounded up to 256 bytes.  0 on invalid arguments.  Pure host function. */
H3DIT_API size_t h3_denoise_workspace_size(const h3_dims* dims, const h3_io_dims* io_dims,
                                          const h3_segments* segments);

H3DIT_API h3_status h3_denoise(const h3_dims* dims, const h3_io_dims* io_dims,
                               const h3_io_weights* io_weights, const h3_segments* segments,
                               const uint16_t* text, const float* cond, float* audio, float* video,
                               const int32_t* tag, const float* positions,
                               const uint16_t* mod_tables, const h3_block_weights* weights,
                               int32_t n_blocks, const uint16_t* final_tables,
                               const double* sigmas_audio, const double* sigmas_video,
                               int32_t n_steps, int32_t reuse, float* x_packed, void* workspace,
                               size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* H3DIT_H */
