/*
 * kvq.h: C ABI of a gfx950 (MI355X) library for attention of a few
 * non-causal queries over a KV cache stored as symmetric group-quantized,
 * nibble-packed 4-bit (or byte-wide 8-bit) codes.
 *
 * Pages describing the method, cited below by tag:
 *   [BKD] "Block KV decoding: less workspace, more time"
 *         (huhohoo.com/en/docs/llm/kv-block-decode-cost)
 *   [KPG] "KV分组打包：4-bit到底省了多少？" (huhohoo.com/docs/llm/kv-packed-groups)
 *   [TOS] "注意力分塊：不保存完整分數矩陣，如何保持結果？"
 *         (huhohoo.com/zh-TW/docs/llm/tiled-online-softmax)
 *   [RL]  "给长前缀列一张有单位的资源账本" (codingai-lec05.pages.dev, resource-ledger)
 *
 * Packed format ([KPG] "what a byte holds", "why grouping needs both
 * direction and length"):
 *   - each group of `group` elements has one float32 scale max|x|/qmax
 *     (qmax = 7 for 4-bit, 127 for 8-bit); a scale that comes out 0 is 1;
 *   - codes are rint(x/scale) (round half to even, IEEE float32 division)
 *     clipped to [-qmax, qmax] and stored unsigned as code + qmax;
 *   - 4-bit: a byte holds two neighbouring elements of one group, the
 *     lower-indexed in the low nibble; 8-bit: one byte per code;
 *   - K ([B,H,N,D] float32) is grouped along tokens inside each channel,
 *     V ([B,H,N,D] float32) along features inside each token; padding
 *     elements are zeros before quantization (stored code = qmax).
 *
 * Byte layout (the pages fix the groups and the byte contents, not the byte
 * order; this one lets the kernels read whole 32-token blocks with
 * contiguous loads that land in registers in matrix-core operand order).
 * Per (b, h): nblocks = ceil(N/32) blocks of 32 tokens; every position that
 * holds no element (token >= N, channel >= D, feature past the last group)
 * stores the zero code qmax.  With kcols = 32*bits/8, D8 = ceil(D/8),
 * Dpad = D rounded up to `group` and vcols = Dpad*bits/8:
 *   K codes  [B][H][nblocks][D8*kcols*8] uint8: in a block, byte
 *            (o*kcols + j)*8 + e holds channel 8o+e of byte column j; a
 *            4-bit column j holds tokens 2j (low nibble) and 2j+1 (high),
 *            an 8-bit column j token j.
 *   K scales [B][H][ceil(N/group)][D] float32 (group-major).
 *   V codes  [B][H][nblocks][4*vcols*8] uint8: in a block, byte
 *            (o*vcols + f)*8 + e holds token 8o+e (o < 4) of byte column f;
 *            a 4-bit column f holds features 2f (low) and 2f+1 (high), an
 *            8-bit column f feature f.
 *   V scales [B][H][nblocks][Dpad/group][32] float32 (token-minor; tokens
 *            >= N carry scale 1, the scale of an all-zero group).
 *
 * Conventions for every call:
 *   - All array pointers are DEVICE pointers to dense row-major arrays in
 *     the layouts above; `stream` is a hipStream_t (NULL = the null stream).
 *     Calls enqueue work on `stream` and return without synchronizing.
 *   - The caller owns and allocates every buffer, including the attention
 *     workspace; the library allocates no memory.
 *   - Arguments are checked before any work is enqueued.  On failure
 *     nothing is written and a negative kvq_status is returned;
 *     kvq_last_error() then holds a message for the calling thread.
 *   - float pointers must be 4-byte aligned.
 *   - Device faults are not reported by these calls; they surface at the
 *     caller's next synchronization, as with any HIP launch.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvq_status {
  KVQ_OK = 0,
  KVQ_ERR_INVALID = -1,     /* null pointer, size < 1, bad format, alias, misalignment */
  KVQ_ERR_UNSUPPORTED = -2, /* valid but not compiled: e.g. attend head dim outside {32,64,128} */
  KVQ_ERR_HIP = -3,         /* the HIP runtime rejected a launch */
  KVQ_ERR_WORKSPACE = -4    /* workspace missing or smaller than kvq_attend_workspace_bytes */
} kvq_status;

/* Attention kernel families for kvq_attend_variant. */
typedef enum kvq_variant {
  KVQ_VARIANT_AUTO = 0,  /* what kvq_attend uses */
  KVQ_VARIANT_VALU = 1,  /* any supported format: decode a tile to float32 in LDS */
  KVQ_VARIANT_MFMA = 2,  /* 4- or 8-bit, group 32, D = 128, <= 32 query rows per KV
                            head: fp16 matrix cores on exact codes */
  KVQ_VARIANT_STREAM = 3 /* 4- or 8-bit, group 8/16/32/64/128, D = 128, <= 8 query rows
                            per KV head: float32 registers, each block read once */
} kvq_variant;

/* Flags of kvq_attend_cache. */
typedef enum kvq_attend_flags {
  KVQ_ATTEND_CAUSAL = 1  /* the R queries of each head are the sequence's last R positions:
                            query r (position N-R+r) reads tokens j <= N-R+r */
} kvq_attend_flags;

/* ---- size limits (every call) -------------------------------------------------
 * N (and capacity) <= 2^31 - 1 - 2^16 tokens, D <= 2^24 and group <= 2^16:
 * larger values make the 32-bit layout arithmetic overflow and are rejected
 * with KVQ_ERR_INVALID (the sizing calls return 0). */

/* ---- host-only sizing (no device work, never fails) ------------------------
 * Byte / element counts of the packed arrays ([KPG] "how to know the file
 * really stores 4-bit": codes plus one float32 scale per group, in the
 * layouts above); 0 if an argument is invalid (size < 1, bits not 4 or 8,
 * group odd or < 2, a size past the limits above). */
size_t kvq_k_code_bytes(int B, int H, int N, int D, int bits, int group);  /* B*H*nblocks*D8*32*bits */
size_t kvq_k_scale_count(int B, int H, int N, int D, int bits, int group); /* B*H*ceil(N/group)*D */
size_t kvq_v_code_bytes(int B, int H, int N, int D, int bits, int group);  /* B*H*nblocks*32*Dpad*bits/8 */
size_t kvq_v_scale_count(int B, int H, int N, int D, int bits, int group); /* B*H*nblocks*(Dpad/group)*32 */

/* Upper bound on the KV splits kvq_attend uses when num_splits == 0, and the
 * split count that sizes the workspace ([RL] "two stops of the online
 * accumulation": per-split (m, z, u) are composable).  The general kernel
 * uses exactly this many; the matrix-core kernel may use fewer. */
int kvq_attend_auto_splits(int B, int Hkv, int N);

/* Workspace bytes kvq_attend / kvq_attend_f32 need for `num_splits` splits
 * (0 = auto: kvq_attend_auto_splits(B, Hkv, N)).  Holds one arrival
 * counter per (batch, KV head), 256 bytes apart at the start, then the
 * per-split partial (m, z, u) of every query row.  The counters must be zero
 * when a call starts and every completed call leaves them zero, whatever its
 * split count: ZERO-FILL a workspace once before its first use, and again
 * before a call with more (batch, KV head) pairs than any earlier call on it
 * (its counters would reach into earlier partials).  Calls that run at the
 * same time must use different workspaces.  A call that finds a head's
 * counter already at or above its split count (a workspace that was not
 * zero-filled as required) cannot trust any ticket: it writes NaN to that
 * head's output rows instead of a merge, and leaves the counter non-zero, so
 * the error shows until the workspace is zero-filled.  (A counter left at a
 * small non-zero value below the split count cannot be told from a live one.) */
size_t kvq_attend_workspace_bytes(int B, int Hq, int Hkv, int R, int N, int D, int num_splits);

/* ---- kvq_pack_k / kvq_pack_v ------------------------------------------------
 * Quantize and pack float32 K or V [B][H][N][D] into codes + scales in the
 * layouts above ([KPG] "what a byte holds"; K and V group along different
 * axes per [KPG] "why grouping needs both direction and length").  Any
 * N, D >= 1 (ragged final groups are zero-padded).  Bit-exact: the scale is
 * one IEEE float32 division, codes one float32 division and rint. */
kvq_status kvq_pack_k(const float* k, int B, int H, int N, int D, int bits, int group,
                      uint8_t* codes, float* scales, void* stream);
kvq_status kvq_pack_v(const float* v, int B, int H, int N, int D, int bits, int group,
                      uint8_t* codes, float* scales, void* stream);

/* ---- kvq_dequant_k / kvq_dequant_v --------------------------------------------
 * Decode the whole packed cache back to float32 [B][H][N][D], cropping the
 * padding: out = fl32((stored - qmax) * scale), one float32 multiply ([KPG]
 * "what a byte holds").  The decode-everything half of the baseline in
 * [BKD] "Compare equivalent representations first".  N * D must be below
 * 2^32 (KVQ_ERR_UNSUPPORTED otherwise). */
kvq_status kvq_dequant_k(const uint8_t* codes, const float* scales, int B, int H, int N, int D,
                         int bits, int group, float* out, void* stream);
kvq_status kvq_dequant_v(const uint8_t* codes, const float* scales, int B, int H, int N, int D,
                         int bits, int group, float* out, void* stream);

/* ---- growing cache: kvq_cache_clear, kvq_append, kvq_attend_cache -------------
 * A decode step reads the cached K/V and appends its new position ([RL]
 * "prefill and decode").  A cache sized for `capacity` tokens uses the
 * layouts above with N = capacity (sizes: kvq_k_code_bytes(B, H, capacity,
 * ...) etc.).  After n tokens it holds exactly the bytes kvq_pack_k/_v write
 * for those n tokens zero-padded to `capacity` ([KPG] "why grouping needs
 * both direction and length": short groups are padded with zeros): positions
 * past n hold the zero code, and K groups past the last token and V groups
 * of tokens past n have scale 1.  V groups lie inside one token, so a new
 * token's V is packed on its own; K groups run along tokens, so the open K
 * group (the one holding token n-1 while n % group != 0) is requantized from
 * float32 whenever tokens join it, its earlier tokens' K taken from k_tail.
 *
 * kvq_cache_clear: the empty cache (n = 0): every stored code qmax, every
 *   scale 1.  k_tail needs no initialization.
 * kvq_append: append T >= 1 tokens k_new, v_new [B][H][T][D] float32 after
 *   the first N >= 0 tokens (N + T <= capacity).  k_tail [B][H][group][D]
 *   float32, slot t % group = K of token t of the open group: read for the
 *   open group's earlier tokens and rewritten for the new open group, so it
 *   must be the tail the previous appends left (unused when N % group == 0).
 *   The cache must hold the state of N tokens (kvq_cache_clear, then appends
 *   of N tokens in total; a prompt can be appended in one call).  Bit-exact:
 *   afterwards the arrays equal the pack of all N + T tokens as above.  The
 *   new rows must not overlap the cache arrays; calls on one cache must be
 *   ordered (one stream).
 * kvq_attend_cache: kvq_attend_variant over the first N tokens of a cache
 *   laid out for `capacity` >= N tokens whose positions past N are in the
 *   empty state above (as kvq_cache_clear + kvq_append leave them).  The
 *   matrix-core limits of kvq_attend_variant apply with capacity in place
 *   of N; capacity == N and flags == 0 is exactly kvq_attend_variant.
 *   flags: 0 or KVQ_ATTEND_CAUSAL, a causal chunk (a prefill chunk or a
 *   multi-token decode step whose R queries were just appended): query r of
 *   each head reads only tokens j <= N-R+r; masked tokens enter neither the
 *   running max nor the sums, and a query with no legal key (N-R+r < 0)
 *   gets zeros ([RL] "why FlashAttention need not keep the whole heat
 *   map").  With R == 1 the flag changes nothing.  Every kernel family
 *   takes the flag. */
kvq_status kvq_cache_clear(int B, int H, int capacity, int D, int bits, int group,
                           uint8_t* k_codes, float* k_scales, uint8_t* v_codes, float* v_scales,
                           void* stream);
kvq_status kvq_append(const float* k_new, const float* v_new, int B, int H, int N, int T,
                      int capacity, int D, int bits, int group, uint8_t* k_codes, float* k_scales,
                      uint8_t* v_codes, float* v_scales, float* k_tail, void* stream);
kvq_status kvq_attend_cache(const float* q, const uint8_t* k_codes, const float* k_scales,
                            const uint8_t* v_codes, const float* v_scales, int B, int Hq, int Hkv,
                            int R, int N, int capacity, int D, int bits, int group,
                            float sm_scale, int num_splits, void* workspace,
                            size_t workspace_bytes, float* out, int variant, int flags,
                            void* stream);

/* ---- kvq_append_attend: one decode step ---------------------------------------------
 * A decode step of [RL] "prefill and decode" (read the cached K/V, append the
 * new position) in one call: kvq_append of one token per KV head (k_new,
 * v_new [B][Hkv][1][D] float32) after the first N >= 0 tokens of the cache,
 * then kvq_attend_cache (variant auto, flags 0) of q over the N + 1 tokens.
 * The cache arrays, k_tail and out end bit for bit as after those two calls.
 * Argument rules are theirs (N + 1 <= capacity; out must not overlap the new
 * rows, k_tail or the workspace).  When the 4-row matrix-core kernel serves
 * the attend (4- or 8-bit, group 32, D = 128, at most 4 query rows per KV
 * head) and a workspace of kvq_attend_workspace_bytes(B, Hq, Hkv, R, N + 1,
 * D, num_splits) bytes is given, both run in one launch: B * Hkv extra
 * workgroups requantize the open K group and pack the token's V with
 * device-scope stores and then raise a flag in the head's counter slot of the
 * workspace, which the one wave attending the token's block waits for (a
 * bounded wait; if it ran out, that head's output would be NaN).  Otherwise
 * the two launches run back to back.  Workspace rules as for kvq_attend (the
 * flag is back at zero after every completed call).  Asynchronous on
 * `stream`. */
kvq_status kvq_append_attend(const float* q, const float* k_new, const float* v_new, int B,
                             int Hq, int Hkv, int R, int N, int capacity, int D, int bits,
                             int group, uint8_t* k_codes, float* k_scales, uint8_t* v_codes,
                             float* v_scales, float* k_tail, float sm_scale, int num_splits,
                             void* workspace, size_t workspace_bytes, float* out, void* stream);

/* ---- kvq_attend ---------------------------------------------------------------
 * out[b][hq][r][:] = softmax_j(sm_scale * q[b][hq][r] . k_j) v_j over all N
 * tokens of KV head hq / (Hq/Hkv), with k_j, v_j decoded from the packed
 * cache inside the kernel ([RL] "GQA changes the shared interface"; no
 * causal mask, [TOS] opening section).  The kernel runs the blocked online
 * softmax of [BKD] "Do not average independently normalized blocks" and
 * [RL] "why FlashAttention need not keep the whole heat map": per query row
 * it carries the running max m, exponential sum z and unnormalized value sum
 * u, rescaling both z and u by exp(m_old - m_new) on every block; KV splits
 * are merged with the same rescale.
 *   q      [B][Hq][R][D] float32          out [B][Hq][R][D] float32
 *   k_codes/k_scales, v_codes/v_scales: the packed layouts above, H = Hkv.
 *   sm_scale: softmax temperature; 0 means 1/sqrt(D) ([RL] "prefill and decode").
 *   num_splits: KV splits; 0 = automatic (at most kvq_attend_auto_splits).
 *   workspace: device buffer of >= kvq_attend_workspace_bytes(...) bytes,
 *     zero-filled before first use (may be NULL only when one split is used).
 * Supported: D in {32, 64, 128}; (Hq/Hkv)*R <= 64; any N >= 1.
 * `out` must not overlap any input.  Accuracy: float32 accumulation, aimed
 * at 1e-4 absolute of a float64 evaluation over the same decoded cache for
 * unit-variance inputs. */
kvq_status kvq_attend(const float* q, const uint8_t* k_codes, const float* k_scales,
                      const uint8_t* v_codes, const float* v_scales,
                      int B, int Hq, int Hkv, int R, int N, int D, int bits, int group,
                      float sm_scale, int num_splits, void* workspace, size_t workspace_bytes,
                      float* out, void* stream);

/* Same contract as kvq_attend with an explicit kernel family.
 * KVQ_VARIANT_MFMA returns KVQ_ERR_UNSUPPORTED unless bits is 4 or 8,
 * group == 32, D == 128, (Hq/Hkv)*R <= 32, N <= 2^25 - 32 (4-bit) or
 * N <= 2^24 - 32 (8-bit) and q and all four cache arrays are 16-byte
 * aligned; KVQ_VARIANT_AUTO picks it whenever those hold.
 * KVQ_VARIANT_STREAM returns KVQ_ERR_UNSUPPORTED unless bits is 4 or 8,
 * group is 8, 16, 32, 64 or 128, D == 128, (Hq/Hkv)*R <= 8, the same N
 * limits hold and the same arrays are 16-byte aligned; KVQ_VARIANT_AUTO
 * picks it where those hold and the matrix-core kernels do not apply.
 * Every other case runs KVQ_VARIANT_VALU. */
kvq_status kvq_attend_variant(const float* q, const uint8_t* k_codes, const float* k_scales,
                              const uint8_t* v_codes, const float* v_scales,
                              int B, int Hq, int Hkv, int R, int N, int D, int bits, int group,
                              float sm_scale, int num_splits, void* workspace,
                              size_t workspace_bytes, float* out, int variant, void* stream);

/* ---- kvq_attend_noalloc --------------------------------------------------------------
 * For callers that cannot allocate memory: code under stream capture, tight
 * serving loops, harnesses that forbid hipMalloc.  kvq_attend with the same
 * arguments except the workspace: the split partials and arrival counters go
 * to a scratch array of 16 MiB that the library keeps in device memory (one
 * copy per GPU, held until the process ends; its address is looked up once
 * per device, on the device's first call).  The call allocates nothing.  It
 * fails with KVQ_ERR_WORKSPACE, before enqueuing anything, when the splits
 * need more than 16 MiB (kvq_attend_workspace_bytes(...) > 16 MiB, e.g. 16
 * splits of 4096 query rows of D = 128).  When the call has more (batch, KV
 * head) pairs than the previous call on this GPU, a small kernel first zeroes
 * the counters that the previous call's partials overwrote.  All calls on one
 * GPU share the scratch: calls that can overlap on one GPU (other streams,
 * other host threads) race and must not be issued. */
kvq_status kvq_attend_noalloc(const float* q, const uint8_t* k_codes, const float* k_scales,
                              const uint8_t* v_codes, const float* v_scales,
                              int B, int Hq, int Hkv, int R, int N, int D, int bits, int group,
                              float sm_scale, int num_splits, float* out, void* stream);

/* ---- kvq_attend_window ------------------------------------------------------------
 * Attention over a mixed cache: N >= 0 packed tokens (the first N tokens of
 * a cache laid out for `capacity` >= max(N, 1) tokens, as kvq_attend_cache
 * reads them) followed by the W >= 1 most recent tokens kept in float32,
 * k_win, v_win [B][Hkv][W][D] ([KPG] "exercises and common mistakes": high
 * precision reserved for the most recent tokens, the packed format
 * unchanged).  The N + W tokens are attended as one sequence: q, out,
 * sm_scale, splits, workspace (sized for N + W tokens) and flags
 * (KVQ_ATTEND_CAUSAL: positions counted over N + W) as in kvq_attend_cache.
 * When the packed part suits the matrix-core kernels (KVQ_VARIANT_MFMA's
 * conditions with capacity for N), or else the streaming kernel
 * (KVQ_VARIANT_STREAM's), the workspace holds S + P split slots,
 * 1 <= P <= ceil(W / 32) (kvq_attend_workspace_bytes(B, Hq, Hkv, R, N + W, D,
 * S + P); S = num_splits, or that kernel's own automatic count, at most
 * kvq_attend_auto_splits(B, Hkv, N)), and k_win and v_win are 16-byte
 * aligned (the window rows are read with 16-byte loads), the call is fused into
 * one launch of that kernel: per KV head, S workgroups attend the packed tokens
 * and P more the window tokens (P the largest count the workspace holds: one
 * workgroup per 32 window tokens at P = ceil(W / 32)), and the split combine
 * merges all S + P partials.  Otherwise the general kernel reads both
 * parts.  A decode
 * loop moves the window's oldest tokens into the packed cache with
 * kvq_append. */
kvq_status kvq_attend_window(const float* q, const uint8_t* k_codes, const float* k_scales,
                             const uint8_t* v_codes, const float* v_scales, const float* k_win,
                             const float* v_win, int B, int Hq, int Hkv, int R, int N, int W,
                             int capacity, int D, int bits, int group, float sm_scale,
                             int num_splits, void* workspace, size_t workspace_bytes, float* out,
                             int flags, void* stream);

/* ---- kvq_attend_f32 -------------------------------------------------------------
 * The same attention over an unquantized float32 cache k, v [B][Hkv][N][D]:
 * the float32-cache reference of [BKD] "Compare equivalent representations
 * first", and, after kvq_dequant_k/_v, the attend half of the decode-all
 * baseline.  Workspace rules as for kvq_attend. */
kvq_status kvq_attend_f32(const float* q, const float* k, const float* v,
                          int B, int Hq, int Hkv, int R, int N, int D, float sm_scale,
                          int num_splits, void* workspace, size_t workspace_bytes, float* out,
                          void* stream);

/* ---- kvq_stream_read ------------------------------------------------------------------
 * Measurement aid, not part of the method: reads `bytes` (a positive multiple
 * of 16) at device pointer `data` (16-byte aligned) once, one contiguous chunk
 * per workgroup with 16-byte nontemporal loads spread over the whole chip
 * (the fastest plain read shape measured on MI355X), and discards them
 * (`sink`: a device word that is
 * written only if the XOR of all the data equals an arbitrary constant).  The
 * fused attend reads every KV byte once ([BKD] "every position is still
 * read"), so this plain read of the same byte count is its measured HBM
 * ceiling.  Allocates nothing; asynchronous on `stream`. */
kvq_status kvq_stream_read(const void* data, size_t bytes, void* sink, void* stream);

/* ---- kvq_phase_trace_fetch -----------------------------------------------------------
 * Measurement aid, not part of the method: the timeline of the last
 * launch of a fused attend kernel, to split its time into the steps of
 * [BKD] "Do not average independently normalized blocks" (stream the blocks,
 * merge partial statistics) and the two stops of [RL] "two stops of the
 * online accumulation" (waves, then KV splits).  Only a library built with
 * KVQ_PHASE_TRACE records anything (quantized_kv_cache_attend_amd/build.py
 * --phase-trace writes it as libkvq_phase.so beside libkvq.so): there every
 * wave of the 4-row (kernel 0) or 32-row (kernel 1) matrix-core kernel or of
 * the streaming kernel (kernel 2) writes the chip-wide 100 MHz clock at
 * KVQ_PHASE_MARKS fixed points
 * (start, query ready, first block ready [not the 32-row kernel], last block done,
 * workgroup merged, partial stores acknowledged, ticket taken, end) for the
 * first KVQ_PHASE_WAVES waves in launch order (workgroup, then wave).  This
 * copies up to `bytes` (a positive multiple of 8) of those uint64 records
 * into host memory `host`, KVQ_PHASE_MARKS per wave; a mark a wave did not
 * reach keeps an older value.  Synchronous.  KVQ_ERR_UNSUPPORTED in the normal
 * build. */
#define KVQ_PHASE_WAVES 16384
#define KVQ_PHASE_MARKS 8
kvq_status kvq_phase_trace_fetch(int kernel, void* host, size_t bytes);

/* ---- diagnostics -------------------------------------------------------------------- */
const char* kvq_status_string(int status);  /* static string, never NULL */
const char* kvq_last_error(void);           /* message of this thread's last failed call */
int kvq_abi_version(void);                  /* bumped on any change of this header */

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
