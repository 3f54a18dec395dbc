// Host side of the C ABI declared in include/kvq.h: argument checks,
// workspace carving, split and kernel selection, launches.  No allocation,
// no synchronization, no global mutable state except a thread-local error
// message.
#include "kvq.h"
#include "kvq_internal.h"
#include "kvq_layout.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>

namespace kvq {
namespace {

thread_local char g_last_error[512] = "";

kvq_status fail(kvq_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

kvq_status ok() {
  g_last_error[0] = '\0';
  return KVQ_OK;
}

// Size limits that keep the layout arithmetic (32-bit ints in make_layout)
// from overflowing: tokens + group and D rounded up to the group stay below
// 2^31, and D * bits / 8 well below it.
constexpr int kMaxGroup = 1 << 16;
constexpr int kMaxTokens = 0x7fffffff - (1 << 16);
constexpr int kMaxDim = 1 << 24;

bool format_ok(int bits, int group) {
  return (bits == 4 || bits == 8) && group >= 2 && group % 2 == 0 && group <= kMaxGroup;
}

bool sizes_in_range(int N, int D) { return N <= kMaxTokens && D <= kMaxDim; }

long long round_up(long long x, long long m) { return (x + m - 1) / m * m; }

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

// [a, a+na) and [b, b+nb) overlap (byte ranges).
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

kvq_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(KVQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

WorkspaceLayout workspace_layout(int B, int Hq, int Hkv, int R, int D, int splits) {
  const size_t rows = static_cast<size_t>(B) * Hq * R;  // every query row once
  WorkspaceLayout w;
  // The arrival counters come first: where they sit depends on the number of
  // (batch, KV head) pairs alone, not on the split count or the row shape.
  w.cnt_off = 0;
  w.m_off = round_up(sizeof(unsigned) * kCounterStride * static_cast<size_t>(B) * Hkv, 256);
  w.z_off = round_up(w.m_off + sizeof(float) * splits * rows, 256);
  w.u_off = round_up(w.z_off + sizeof(float) * splits * rows, 256);
  w.total = round_up(w.u_off + sizeof(float) * splits * rows * D, 256);
  return w;
}

}  // namespace kvq

using namespace kvq;

namespace {

int auto_splits(int B, int Hkv, int N) {
  // About 512 workgroups: two per compute unit, all resident at once, so
  // every KV byte's load can be in flight early.  A split is at least one
  // 32-token tile: a workgroup walks its tiles one after another (each a
  // load, a decode and the math, ~4 us), so a short cache on few heads is
  // fastest spread one tile per workgroup.
  const long long heads = static_cast<long long>(B) * Hkv;
  const long long want = (512 + heads - 1) / heads;
  const long long cap = (N + kBlockTokens - 1) / kBlockTokens;
  long long s = want < cap ? want : cap;
  if (s < 1) s = 1;
  if (s > 1024) s = 1024;
  return static_cast<int>(s);
}

// Shared validation of the attention calls.  `bits` == 32 marks the
// float32-cache path.
// `cap`: tokens the packed layout is sized for (>= the n_packed tokens read
// from it; N for the float32 cache).  N counts every token attended.
kvq_status check_attend(const float* q, const void* k, const void* ks, const void* v,
                        const void* vs, int B, int Hq, int Hkv, int R, int N, int cap, int D,
                        int bits, int group, float sm_scale, int num_splits, void* workspace,
                        size_t workspace_bytes, float* out, AttendProblem* p, int n_packed = -1) {
  if (n_packed < 0) n_packed = N;
  if (!q || !k || !v || !out || (bits != 32 && (!ks || !vs)))
    return fail(KVQ_ERR_INVALID, "null pointer argument");
  if (B < 1 || Hq < 1 || Hkv < 1 || R < 1 || N < 1 || D < 1)
    return fail(KVQ_ERR_INVALID, "sizes must be >= 1 (B=%d Hq=%d Hkv=%d R=%d N=%d D=%d)", B, Hq,
                Hkv, R, N, D);
  if (!sizes_in_range(N, D) || cap > kMaxTokens)
    return fail(KVQ_ERR_INVALID, "N=%d / capacity=%d above %d tokens or D=%d above %d", N, cap,
                kMaxTokens, D, kMaxDim);
  if (Hq % Hkv) return fail(KVQ_ERR_INVALID, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (cap < n_packed || cap < 1)
    return fail(KVQ_ERR_INVALID, "capacity=%d < %d packed tokens", cap, n_packed);
  if (bits != 32 && !format_ok(bits, group))
    return fail(KVQ_ERR_INVALID, "format bits=%d group=%d (need bits 4|8, even group in [2, %d])",
                bits, group, kMaxGroup);
  if (num_splits < 0) return fail(KVQ_ERR_INVALID, "num_splits=%d < 0", num_splits);
  if (!(std::isfinite(sm_scale)) || sm_scale < 0.0f)
    return fail(KVQ_ERR_INVALID, "sm_scale must be finite and >= 0");
  if (!aligned(q, 4) || !aligned(out, 4) || (bits != 32 && (!aligned(ks, 4) || !aligned(vs, 4))) ||
      (bits == 32 && (!aligned(k, 4) || !aligned(v, 4))))
    return fail(KVQ_ERR_INVALID, "float arrays must be 4-byte aligned");
  if (D != 32 && D != 64 && D != 128)
    return fail(KVQ_ERR_UNSUPPORTED, "head dim D=%d not in {32, 64, 128}", D);
  const int rows = (Hq / Hkv) * R;
  if (rows > kMaxRows)
    return fail(KVQ_ERR_UNSUPPORTED, "(Hq/Hkv)*R = %d query rows per KV head > %d", rows,
                kMaxRows);

  const long long BH = static_cast<long long>(B) * Hkv;
  const size_t out_bytes = sizeof(float) * static_cast<size_t>(B) * Hq * R * D;
  size_t kb, vb, ksb = 0, vsb = 0;
  if (bits == 32) {
    kb = vb = sizeof(float) * static_cast<size_t>(BH) * N * D;
  } else {
    const Layout L = make_layout(cap, D, bits, group);
    kb = static_cast<size_t>(BH * k_code_bytes_per_head(L));
    vb = static_cast<size_t>(BH * v_code_bytes_per_head(L));
    ksb = sizeof(float) * static_cast<size_t>(BH * k_scales_per_head(L));
    vsb = sizeof(float) * static_cast<size_t>(BH * v_scales_per_head(L));
  }
  if (overlaps(out, out_bytes, q, out_bytes) || overlaps(out, out_bytes, k, kb) ||
      overlaps(out, out_bytes, v, vb) || (ksb && overlaps(out, out_bytes, ks, ksb)) ||
      (vsb && overlaps(out, out_bytes, vs, vsb)))
    return fail(KVQ_ERR_INVALID, "out overlaps an input");

  const int splits = num_splits ? num_splits : auto_splits(B, Hkv, N);
  if (splits > 65535) return fail(KVQ_ERR_INVALID, "num_splits=%d > 65535", splits);
  const WorkspaceLayout wl = workspace_layout(B, Hq, Hkv, R, D, splits);
  if (splits > 1) {
    if (!workspace) return fail(KVQ_ERR_WORKSPACE, "%d splits need a workspace", splits);
    if (workspace_bytes < wl.total)
      return fail(KVQ_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes,
                  wl.total);
    if (!aligned(workspace, 16)) return fail(KVQ_ERR_INVALID, "workspace must be 16-byte aligned");
    if (overlaps(out, out_bytes, workspace, wl.total))
      return fail(KVQ_ERR_INVALID, "out overlaps the workspace");
  }

  p->q = q;
  p->k_codes = static_cast<const uint8_t*>(k);
  p->k_scales = static_cast<const float*>(ks);
  p->v_codes = static_cast<const uint8_t*>(v);
  p->v_scales = static_cast<const float*>(vs);
  p->k_f32 = static_cast<const float*>(k);
  p->v_f32 = static_cast<const float*>(v);
  p->out = out;
  p->B = B;
  p->Hq = Hq;
  p->Hkv = Hkv;
  p->R = R;
  p->N = N;
  p->cap = cap;
  p->causal = 0;
  p->k_win = p->v_win = nullptr;
  p->W = 0;
  p->win_parts = 0;
  p->win_per_part = 0;
  p->pos_end = N;
  p->D = D;
  p->rows = rows;
  p->bits = bits;
  p->group = bits == 32 ? 1 : group;
  const float scale = sm_scale > 0.0f ? sm_scale : 1.0f / std::sqrt(static_cast<float>(D));
  p->qscale = scale * kLog2e;
  p->splits = splits;
  p->spw = 1;
  p->tokens_per_split =
      static_cast<int>(round_up((static_cast<long long>(N) + splits - 1) / splits, kBlockTokens));
  p->codes_aligned = bits != 32 && aligned(k, 4) && aligned(v, 4);
  char* ws = static_cast<char*>(workspace);
  p->part_m = splits > 1 ? reinterpret_cast<float*>(ws + wl.m_off) : nullptr;
  p->part_z = splits > 1 ? reinterpret_cast<float*>(ws + wl.z_off) : nullptr;
  p->part_u = splits > 1 ? reinterpret_cast<float*>(ws + wl.u_off) : nullptr;
  p->counters = splits > 1 ? reinterpret_cast<unsigned*>(ws + wl.cnt_off) : nullptr;
  p->append = 0;
  p->k_new = p->v_new = nullptr;
  p->k_tail = nullptr;
  p->k_codes_w = p->v_codes_w = nullptr;
  p->k_scales_w = p->v_scales_w = nullptr;
  return KVQ_OK;
}

// The matrix-core kernels address a head's arrays with 32-bit buffer
// offsets below 2^31: fewer than 2^20 blocks of 2 KB (4-bit) or 2^19 blocks
// of 4 KB (8-bit) per head.
constexpr int kMfmaMaxN = (1 << 25) - kBlockTokens;
constexpr int kMfmaMaxN8 = (1 << 24) - kBlockTokens;

bool mfma_eligible(const AttendProblem& p) {
  return (p.bits == 4 || p.bits == 8) && p.group == 32 && p.D == 128 &&
         p.rows <= kMfma32MaxRows && p.cap <= (p.bits == 8 ? kMfmaMaxN8 : kMfmaMaxN) &&
         aligned(p.q, 16) && aligned(p.k_codes, 16) && aligned(p.v_codes, 16) &&
         aligned(p.k_scales, 16) && aligned(p.v_scales, 16);
}

// Split count of the matrix-core kernel when the caller asks for auto: one
// 8-wave workgroup per compute unit (about 256 workgroups; every split is
// merged by the fused tail, so fewer, larger splits are cheaper once the
// compute units are covered), and no split shorter than 1024 tokens.  Never
// more than auto_splits(), so a workspace sized by
// kvq_attend_workspace_bytes(..., 0) always suffices.
int mfma_auto_splits(int B, int Hkv, int N) {
  const long long heads = static_cast<long long>(B) * Hkv;
  const long long want = (256 + heads - 1) / heads;
  const long long cap = (N + 1023) / 1024;
  long long s = want < cap ? want : cap;
  if (s < 1) s = 1;
  const long long general = auto_splits(B, Hkv, N);
  return static_cast<int>(s < general ? s : general);
}

// The 32-row kernel runs 4-wave workgroups, two per compute unit: about 512
// workgroups (one round: a second one costs ~50 %), no split shorter than
// 512 tokens (four blocks per wave).  On the 8 x 4096-token cache with 8 to
// 32 rows per KV head, 8 splits take 18.7-24.7 us where 2 took 27-39 us.
int mfma32_auto_splits(int B, int Hkv, int N) {
  const long long heads = static_cast<long long>(B) * Hkv;
  const long long want = (512 + heads - 1) / heads;
  const long long cap = (N + 511) / 512;
  long long s = want < cap ? want : cap;
  if (s < 1) s = 1;
  const long long general = auto_splits(B, Hkv, N);
  return static_cast<int>(s < general ? s : general);
}

// Splits per workgroup of the 32-row kernel.  When a head's splits would
// fill at least 4 rounds of its 4-wave workgroups (512 a round: two per
// compute unit), each workgroup takes a run of consecutive splits of its head
// (a multiple of 4 splits, so the waves get equal shares): each wave attends
// whole splits of the run, the workgroup merges its waves and stores one
// partial for the run, and the last arriver merges one partial per
// workgroup.  The rounds' start-up and tail are paid once, and a quarter of
// the partial rows or fewer go through memory.  With fewer, one split per
// workgroup.  Not with window parts (the
// whole-split waves take at most two masked blocks, which holds while the
// queries end at N), nor for causal calls with 8-bit codes and more than 16
// rows (that form is not compiled).
int mfma32_splits_per_wg(const AttendProblem& p) {
  constexpr int kWaves = 4;
  if (p.win_parts > 0 || p.pos_end != p.N || p.splits < kWaves) return 1;
  if (p.causal && p.bits == 8 && p.rows > 16) return 1;
  const long long wgs = static_cast<long long>(p.B) * p.Hkv * p.splits;
  const long long per = (wgs + 511) / 512;
  if (per < kWaves) return 1;
  const long long spw = (per + kWaves - 1) / kWaves * kWaves;
  const long long all = (static_cast<long long>(p.splits) + kWaves - 1) / kWaves * kWaves;
  return static_cast<int>(spw < all ? spw : all);
}

hipError_t run_mfma(AttendProblem p, bool auto_split, hipStream_t s) {
  const bool wide = p.rows > kMfmaMaxRows;
  if (auto_split)
    p.splits = wide ? mfma32_auto_splits(p.B, p.Hkv, p.N) : mfma_auto_splits(p.B, p.Hkv, p.N);
  p.tokens_per_split = mfma_tokens_per_split(p.N, p.splits);
  if (wide) p.spw = mfma32_splits_per_wg(p);
  return wide ? launch_attend_mfma32(p, s) : launch_attend_mfma(p, s);
}

// The streaming kernel takes D = 128 and power-of-two groups from 8 to 128
// (a token octet then lies in one K group, and a feature pair in one V
// group; dpad = 128), up to 8 rows, causal or not, no float32 window, with the matrix-core
// kernels' size and alignment conditions (32-bit buffer offsets per head:
// group-8 scales take 64 bytes per token and head).
bool stream_eligible(const AttendProblem& p) {
  const int g = p.group;
  return (p.bits == 4 || p.bits == 8) && g >= 8 && g <= 128 && (g & (g - 1)) == 0 &&
         p.D == 128 && p.rows <= kStreamMaxRows && p.W == 0 &&
         p.cap <= (p.bits == 8 ? kMfmaMaxN8 : kMfmaMaxN) && aligned(p.q, 16) &&
         aligned(p.k_codes, 16) && aligned(p.v_codes, 16) && aligned(p.k_scales, 16) &&
         aligned(p.v_scales, 16);
}

// Split count of the streaming kernel when the caller asks for auto: about
// 2048 waves, two per SIMD (one 8-wave workgroup per compute unit, or two of
// 4 waves), every wave with the same number of blocks, at least one block per
// wave, never more than auto_splits().  On the 8 x 4096-token cache with 32
// query heads over 8 KV heads (4-bit group 8) 4 splits take 24.8 us, 2 take
// 39.9 us and 8 take 33.0 us.
int stream_auto_splits(int B, int Hkv, int N, int waves) {
  const long long heads = static_cast<long long>(B) * Hkv;
  const long long per_head = static_cast<long long>(waves) * heads;
  const long long want = (2048 + per_head - 1) / per_head;
  const long long blocks = (N + kBlockTokens - 1) / kBlockTokens;
  const long long cap = (blocks + waves - 1) / waves;
  long long s = want < cap ? want : cap;
  if (s < 1) s = 1;
  const long long general = auto_splits(B, Hkv, N);
  return static_cast<int>(s < general ? s : general);
}

hipError_t run_stream(AttendProblem p, bool auto_split, hipStream_t s) {
  if (auto_split) {
    p.splits = stream_auto_splits(p.B, p.Hkv, p.N, stream_waves(p.bits, p.rows));
    p.tokens_per_split = static_cast<int>(
        round_up((static_cast<long long>(p.N) + p.splits - 1) / p.splits, kBlockTokens));
  }
  return launch_attend_stream(p, s);
}

// The automatic choice over the packed cache: matrix cores, else the
// streaming kernel, else the general one.
hipError_t run_packed(const AttendProblem& p, bool auto_split, hipStream_t s) {
  if (mfma_eligible(p)) return run_mfma(p, auto_split, s);
  if (stream_eligible(p)) return run_stream(p, auto_split, s);
  return launch_attend_valu(p, s);
}

kvq_status codec_check(const void* a, const void* b, const void* c, int B, int H, int N, int D,
                       int bits, int group) {
  if (!a || !b || !c) return fail(KVQ_ERR_INVALID, "null pointer argument");
  if (B < 1 || H < 1 || N < 1 || D < 1)
    return fail(KVQ_ERR_INVALID, "sizes must be >= 1 (B=%d H=%d N=%d D=%d)", B, H, N, D);
  if (!format_ok(bits, group))
    return fail(KVQ_ERR_INVALID, "format bits=%d group=%d (need bits 4|8, even group in [2, %d])",
                bits, group, kMaxGroup);
  if (!sizes_in_range(N, D))
    return fail(KVQ_ERR_INVALID, "N=%d above %d tokens or D=%d above %d", N, kMaxTokens, D,
                kMaxDim);
  return KVQ_OK;
}

// ---- the library's own scratch memory (kvq_attend_noalloc) -------------------
// For callers that cannot allocate (code under stream capture, tight serving
// loops, harnesses that forbid hipMalloc): a workspace in a file-scope device
// array that each GPU holds until the process ends.  Host code never passes
// the array's name to a kernel (on the host it is only a stand-in for the
// symbol): the device address of each GPU's copy comes from
// hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};
// Bytes at the start of each device's scratch known to be zero: after a call
// on H (batch, KV head) pairs, its 256 * H bytes of arrival counters (the
// partials that follow are garbage to a later call's counters).
size_t g_scratch_clean[kMaxDevices] = {};

__global__ void zero_bytes_kernel(unsigned char* p, size_t n) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
    p[i] = 0;
}

// This device's scratch address, looked up on the device's first call.
kvq_status scratch_address(int* dev_out, void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(KVQ_ERR_UNSUPPORTED, "device %d beyond the %d the scratch table holds", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(KVQ_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
    g_scratch_clean[dev] = 0;  // the first call clears its counters itself
  }
  *dev_out = dev;
  *ptr = g_scratch_ptr[dev];
  return KVQ_OK;
}

// Start of the range [from, need) of a device's scratch that must be zeroed
// before a call whose counters take `need` bytes; afterwards exactly `need`
// bytes are known to be zero.
size_t scratch_claim(int dev, size_t need) {
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  const size_t from = g_scratch_clean[dev] < need ? g_scratch_clean[dev] : need;
  g_scratch_clean[dev] = need;
  return from;
}

}  // namespace

extern "C" {

size_t kvq_k_code_bytes(int B, int H, int N, int D, int bits, int group) {
  if (B < 1 || H < 1 || N < 1 || D < 1 || !format_ok(bits, group) || !sizes_in_range(N, D))
    return 0;
  return static_cast<size_t>(B) * H * k_code_bytes_per_head(make_layout(N, D, bits, group));
}
size_t kvq_k_scale_count(int B, int H, int N, int D, int bits, int group) {
  if (B < 1 || H < 1 || N < 1 || D < 1 || !format_ok(bits, group) || !sizes_in_range(N, D))
    return 0;
  return static_cast<size_t>(B) * H * k_scales_per_head(make_layout(N, D, bits, group));
}
size_t kvq_v_code_bytes(int B, int H, int N, int D, int bits, int group) {
  if (B < 1 || H < 1 || N < 1 || D < 1 || !format_ok(bits, group) || !sizes_in_range(N, D))
    return 0;
  return static_cast<size_t>(B) * H * v_code_bytes_per_head(make_layout(N, D, bits, group));
}
size_t kvq_v_scale_count(int B, int H, int N, int D, int bits, int group) {
  if (B < 1 || H < 1 || N < 1 || D < 1 || !format_ok(bits, group) || !sizes_in_range(N, D))
    return 0;
  return static_cast<size_t>(B) * H * v_scales_per_head(make_layout(N, D, bits, group));
}

int kvq_attend_auto_splits(int B, int Hkv, int N) {
  if (B < 1 || Hkv < 1 || N < 1) return 0;
  return auto_splits(B, Hkv, N);
}

size_t kvq_attend_workspace_bytes(int B, int Hq, int Hkv, int R, int N, int D, int num_splits) {
  if (B < 1 || Hq < 1 || Hkv < 1 || R < 1 || N < 1 || D < 1 || num_splits < 0) return 0;
  const int s = num_splits ? num_splits : auto_splits(B, Hkv, N);
  return workspace_layout(B, Hq, Hkv, R, D, s).total;
}

kvq_status kvq_pack_k(const float* k, int B, int H, int N, int D, int bits, int group,
                      uint8_t* codes, float* scales, void* stream) {
  const kvq_status st = codec_check(k, codes, scales, B, H, N, D, bits, group);
  if (st != KVQ_OK) return st;
  return hip_status(launch_pack(k, B, H, N, D, bits, group, true, codes, scales,
                                static_cast<hipStream_t>(stream)),
                    "pack_k launch");
}

kvq_status kvq_pack_v(const float* v, int B, int H, int N, int D, int bits, int group,
                      uint8_t* codes, float* scales, void* stream) {
  const kvq_status st = codec_check(v, codes, scales, B, H, N, D, bits, group);
  if (st != KVQ_OK) return st;
  return hip_status(launch_pack(v, B, H, N, D, bits, group, false, codes, scales,
                                static_cast<hipStream_t>(stream)),
                    "pack_v launch");
}

kvq_status kvq_dequant_k(const uint8_t* codes, const float* scales, int B, int H, int N, int D,
                         int bits, int group, float* out, void* stream) {
  const kvq_status st = codec_check(codes, scales, out, B, H, N, D, bits, group);
  if (st != KVQ_OK) return st;
  if (static_cast<long long>(N) * D >= (1LL << 32))
    return fail(KVQ_ERR_UNSUPPORTED, "dequant of N * D >= 2^32 elements per head (N=%d D=%d)", N, D);
  return hip_status(launch_dequant(codes, scales, B, H, N, D, bits, group, true, out,
                                   static_cast<hipStream_t>(stream)),
                    "dequant_k launch");
}

kvq_status kvq_dequant_v(const uint8_t* codes, const float* scales, int B, int H, int N, int D,
                         int bits, int group, float* out, void* stream) {
  const kvq_status st = codec_check(codes, scales, out, B, H, N, D, bits, group);
  if (st != KVQ_OK) return st;
  if (static_cast<long long>(N) * D >= (1LL << 32))
    return fail(KVQ_ERR_UNSUPPORTED, "dequant of N * D >= 2^32 elements per head (N=%d D=%d)", N, D);
  return hip_status(launch_dequant(codes, scales, B, H, N, D, bits, group, false, out,
                                   static_cast<hipStream_t>(stream)),
                    "dequant_v launch");
}

kvq_status kvq_cache_clear(int B, int H, int capacity, int D, int bits, int group,
                           uint8_t* k_codes, float* k_scales, uint8_t* v_codes, float* v_scales,
                           void* stream) {
  if (!k_codes || !k_scales || !v_codes || !v_scales)
    return fail(KVQ_ERR_INVALID, "null pointer argument");
  if (B < 1 || H < 1 || capacity < 1 || D < 1)
    return fail(KVQ_ERR_INVALID, "sizes must be >= 1 (B=%d H=%d capacity=%d D=%d)", B, H,
                capacity, D);
  if (!sizes_in_range(capacity, D))
    return fail(KVQ_ERR_INVALID, "capacity=%d above %d tokens or D=%d above %d", capacity,
                kMaxTokens, D, kMaxDim);
  if (!format_ok(bits, group))
    return fail(KVQ_ERR_INVALID, "format bits=%d group=%d (need bits 4|8, even group in [2, %d])",
                bits, group, kMaxGroup);
  if (!aligned(k_scales, 4) || !aligned(v_scales, 4))
    return fail(KVQ_ERR_INVALID, "float arrays must be 4-byte aligned");
  return hip_status(launch_cache_clear(B, H, capacity, D, bits, group, k_codes, k_scales, v_codes,
                                       v_scales, static_cast<hipStream_t>(stream)),
                    "cache_clear launch");
}

}  // extern "C"

namespace {

// Arguments of an append of T tokens after the first N (kvq_append).
kvq_status check_append(const float* k_new, const float* v_new, int B, int H, int N, int T,
                        int capacity, int D, int bits, int group, const uint8_t* k_codes,
                        const float* k_scales, const uint8_t* v_codes, const float* v_scales,
                        const float* k_tail) {
  if (!k_new || !v_new || !k_codes || !k_scales || !v_codes || !v_scales || !k_tail)
    return fail(KVQ_ERR_INVALID, "null pointer argument");
  if (B < 1 || H < 1 || T < 1 || D < 1 || N < 0)
    return fail(KVQ_ERR_INVALID, "sizes must be >= 1, N >= 0 (B=%d H=%d N=%d T=%d D=%d)", B, H,
                N, T, D);
  if (capacity < 1 || static_cast<long long>(N) + T > capacity)
    return fail(KVQ_ERR_INVALID, "N + T = %lld exceeds capacity=%d",
                static_cast<long long>(N) + T, capacity);
  if (!sizes_in_range(capacity, D))
    return fail(KVQ_ERR_INVALID, "capacity=%d above %d tokens or D=%d above %d", capacity,
                kMaxTokens, D, kMaxDim);
  if (!format_ok(bits, group))
    return fail(KVQ_ERR_INVALID, "format bits=%d group=%d (need bits 4|8, even group in [2, %d])",
                bits, group, kMaxGroup);
  if (!aligned(k_new, 4) || !aligned(v_new, 4) || !aligned(k_scales, 4) || !aligned(v_scales, 4) ||
      !aligned(k_tail, 4))
    return fail(KVQ_ERR_INVALID, "float arrays must be 4-byte aligned");
  const long long BH = static_cast<long long>(B) * H;
  const Layout L = make_layout(capacity, D, bits, group);
  const size_t new_bytes = sizeof(float) * static_cast<size_t>(BH) * T * D;
  const size_t tail_bytes = sizeof(float) * static_cast<size_t>(BH) * group * D;
  const void* ins[2] = {k_new, v_new};
  const void* outs[5] = {k_codes, k_scales, v_codes, v_scales, k_tail};
  const size_t out_bytes[5] = {static_cast<size_t>(BH * k_code_bytes_per_head(L)),
                               sizeof(float) * static_cast<size_t>(BH * k_scales_per_head(L)),
                               static_cast<size_t>(BH * v_code_bytes_per_head(L)),
                               sizeof(float) * static_cast<size_t>(BH * v_scales_per_head(L)),
                               tail_bytes};
  for (int a = 0; a < 5; ++a) {
    for (int b = 0; b < 2; ++b)
      if (overlaps(outs[a], out_bytes[a], ins[b], new_bytes))
        return fail(KVQ_ERR_INVALID, "the new K/V rows overlap a cache array");
    for (int b = a + 1; b < 5; ++b)
      if (overlaps(outs[a], out_bytes[a], outs[b], out_bytes[b]))
        return fail(KVQ_ERR_INVALID, "cache arrays overlap");
  }
  return KVQ_OK;
}

}  // namespace

extern "C" {

kvq_status kvq_append(const float* k_new, const float* v_new, int B, int H, int N, int T,
                      int capacity, int D, int bits, int group, uint8_t* k_codes, float* k_scales,
                      uint8_t* v_codes, float* v_scales, float* k_tail, void* stream) {
  const kvq_status st = check_append(k_new, v_new, B, H, N, T, capacity, D, bits, group, k_codes,
                                     k_scales, v_codes, v_scales, k_tail);
  if (st != KVQ_OK) return st;
  return hip_status(launch_append(k_new, v_new, B, H, N, T, capacity, D, bits, group, k_codes,
                                  k_scales, v_codes, v_scales, k_tail,
                                  static_cast<hipStream_t>(stream)),
                    "append launch");
}
kvq_status kvq_attend_cache(const float* q, const uint8_t* k_codes, const float* k_scales,
                            const uint8_t* v_codes, const float* v_scales, int B, int Hq, int Hkv,
                            int R, int N, int capacity, int D, int bits, int group,
                            float sm_scale, int num_splits, void* workspace,
                            size_t workspace_bytes, float* out, int variant, int flags,
                            void* stream) {
  AttendProblem p;
  kvq_status st = check_attend(q, k_codes, k_scales, v_codes, v_scales, B, Hq, Hkv, R, N, capacity,
                               D, bits, group, sm_scale, num_splits, workspace, workspace_bytes,
                               out, &p);
  if (st != KVQ_OK) return st;
  if (flags & ~KVQ_ATTEND_CAUSAL) return fail(KVQ_ERR_INVALID, "unknown flags 0x%x", flags);
  // One query per head reads every token under the causal rule too.
  p.causal = (flags & KVQ_ATTEND_CAUSAL) && R > 1;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  switch (variant) {
    case KVQ_VARIANT_AUTO:
      return hip_status(run_packed(p, num_splits == 0, s), "attend launch");
    case KVQ_VARIANT_VALU:
      return hip_status(launch_attend_valu(p, s), "attend (valu) launch");
    case KVQ_VARIANT_MFMA:
      if (!mfma_eligible(p))
        return fail(KVQ_ERR_UNSUPPORTED,
                    "matrix-core kernels need bits=4|8, group=32, D=128, <= %d query rows per "
                    "KV head, N <= %d (4-bit) or %d (8-bit) and 16-byte aligned q and cache "
                    "arrays", kMfma32MaxRows, kMfmaMaxN, kMfmaMaxN8);
      return hip_status(run_mfma(p, num_splits == 0, s), "attend (mfma) launch");
    case KVQ_VARIANT_STREAM:
      if (!stream_eligible(p))
        return fail(KVQ_ERR_UNSUPPORTED,
                    "the streaming kernel needs bits=4|8, group 8|16|32|64|128, D=128, <= %d "
                    "query rows per KV head, no float32 window, N <= %d (4-bit) or %d (8-bit) and "
                    "16-byte aligned q and cache arrays", kStreamMaxRows, kMfmaMaxN, kMfmaMaxN8);
      return hip_status(run_stream(p, num_splits == 0, s), "attend (stream) launch");
    default:
      return fail(KVQ_ERR_INVALID, "unknown variant %d", variant);
  }
}

kvq_status kvq_append_attend(const float* q, const float* k_new, const float* v_new, int B,
                             int Hq, int Hkv, int R, int N, int capacity, int D, int bits,
                             int group, uint8_t* k_codes, float* k_scales, uint8_t* v_codes,
                             float* v_scales, float* k_tail, float sm_scale, int num_splits,
                             void* workspace, size_t workspace_bytes, float* out, void* stream) {
  if (Hkv < 1 || N < 0) return fail(KVQ_ERR_INVALID, "Hkv=%d < 1 or N=%d < 0", Hkv, N);
  kvq_status st = check_append(k_new, v_new, B, Hkv, N, 1, capacity, D, bits, group, k_codes,
                               k_scales, v_codes, v_scales, k_tail);
  if (st != KVQ_OK) return st;
  AttendProblem p;
  st = check_attend(q, k_codes, k_scales, v_codes, v_scales, B, Hq, Hkv, R, N + 1, capacity, D,
                    bits, group, sm_scale, num_splits, workspace, workspace_bytes, out, &p);
  if (st != KVQ_OK) return st;
  const long long BH = static_cast<long long>(B) * Hkv;
  const size_t out_bytes = sizeof(float) * static_cast<size_t>(B) * Hq * R * D;
  if (overlaps(out, out_bytes, k_new, sizeof(float) * BH * D) ||
      overlaps(out, out_bytes, v_new, sizeof(float) * BH * D) ||
      overlaps(out, out_bytes, k_tail, sizeof(float) * BH * group * D))
    return fail(KVQ_ERR_INVALID, "out overlaps the new rows or k_tail");
  const WorkspaceLayout wl = workspace_layout(B, Hq, Hkv, R, D, p.splits);
  // One launch when the 4-row matrix-core kernel serves the step and the
  // workspace holds the heads' counters (the append flags live there).
  const bool fused = mfma_eligible(p) && p.rows <= kMfmaMaxRows && workspace != nullptr &&
                     aligned(workspace, 16) && workspace_bytes >= wl.total;
  if (fused && overlaps(out, out_bytes, workspace, wl.total))
    return fail(KVQ_ERR_INVALID, "out overlaps the workspace");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (!fused) {
    st = hip_status(launch_append(k_new, v_new, B, Hkv, N, 1, capacity, D, bits, group, k_codes,
                                  k_scales, v_codes, v_scales, k_tail, s),
                    "append launch");
    if (st != KVQ_OK) return st;
    return hip_status(run_packed(p, num_splits == 0, s), "attend launch");
  }
  p.append = 1;
  p.k_new = k_new;
  p.v_new = v_new;
  p.k_tail = k_tail;
  p.k_codes_w = k_codes;
  p.k_scales_w = k_scales;
  p.v_codes_w = v_codes;
  p.v_scales_w = v_scales;
  p.counters = reinterpret_cast<unsigned*>(static_cast<char*>(workspace) + wl.cnt_off);
  return hip_status(run_mfma(p, num_splits == 0, s), "append + attend (mfma) launch");
}

kvq_status kvq_attend_window(const float* q, const uint8_t* k_codes, const float* k_scales,
                             const uint8_t* v_codes, const float* v_scales, const float* k_win,
                             const float* v_win, int B, int Hq, int Hkv, int R, int N, int W,
                             int capacity, int D, int bits, int group, float sm_scale,
                             int num_splits, void* workspace, size_t workspace_bytes, float* out,
                             int flags, void* stream) {
  if (!k_win || !v_win) return fail(KVQ_ERR_INVALID, "null pointer argument");
  if (N < 0 || W < 1 || static_cast<long long>(N) + W > 0x7fffffff)
    return fail(KVQ_ERR_INVALID, "need N >= 0 packed tokens and W >= 1 window tokens (N=%d W=%d)",
                N, W);
  if (!aligned(k_win, 4) || !aligned(v_win, 4))
    return fail(KVQ_ERR_INVALID, "float arrays must be 4-byte aligned");
  if (flags & ~KVQ_ATTEND_CAUSAL) return fail(KVQ_ERR_INVALID, "unknown flags 0x%x", flags);
  AttendProblem p;
  kvq_status st = check_attend(q, k_codes, k_scales, v_codes, v_scales, B, Hq, Hkv, R, N + W,
                               capacity, D, bits, group, sm_scale, num_splits, workspace,
                               workspace_bytes, out, &p, N);
  if (st != KVQ_OK) return st;
  const size_t out_bytes = sizeof(float) * static_cast<size_t>(B) * Hq * R * D;
  const size_t win_bytes = sizeof(float) * static_cast<size_t>(B) * Hkv * W * D;
  if (overlaps(out, out_bytes, k_win, win_bytes) || overlaps(out, out_bytes, v_win, win_bytes))
    return fail(KVQ_ERR_INVALID, "out overlaps the window");
  p.causal = (flags & KVQ_ATTEND_CAUSAL) && R > 1;
  const hipStream_t s = static_cast<hipStream_t>(stream);

  // Fused form, one launch of a matrix-core kernel (or, for the formats it
  // takes, of the streaming kernel): S workgroups per head attend the packed
  // tokens and P more attend the W float32 window tokens (one per 32 tokens
  // when the workspace has the slots); the fused combine merges all S + P
  // partials.  (The fused form reads the window rows with 16-byte loads.)
  if (N >= 1 && aligned(k_win, 16) && aligned(v_win, 16)) {
    AttendProblem pm = p;
    pm.N = N;
    pm.pos_end = N + W;
    const bool mfma = mfma_eligible(pm);
    if (mfma || stream_eligible(pm)) {  // (pm.W is still 0: the packed part alone)
      const bool wide = pm.rows > kMfmaMaxRows;
      const int S = num_splits ? num_splits
                    : !mfma    ? stream_auto_splits(B, Hkv, N, stream_waves(bits, pm.rows))
                               : (wide ? mfma32_auto_splits(B, Hkv, N) : mfma_auto_splits(B, Hkv, N));
      int P = (W + kBlockTokens - 1) / kBlockTokens;  // window parts wanted
      while (P > 1 && (S + P > 65535 || !workspace ||
                       workspace_bytes < workspace_layout(B, Hq, Hkv, R, D, S + P).total))
        --P;
      const WorkspaceLayout wl = workspace_layout(B, Hq, Hkv, R, D, S + P);
      if (S + P <= 65535 && workspace && workspace_bytes >= wl.total) {
        char* ws = static_cast<char*>(workspace);
        pm.splits = S + P;  // S packed splits, then P window parts
        pm.win_parts = P;
        pm.win_per_part = (W + P - 1) / P;
        pm.k_win = k_win;
        pm.v_win = v_win;
        pm.W = W;
        pm.tokens_per_split = mfma_tokens_per_split(N, S);
        pm.part_m = reinterpret_cast<float*>(ws + wl.m_off);
        pm.part_z = reinterpret_cast<float*>(ws + wl.z_off);
        pm.part_u = reinterpret_cast<float*>(ws + wl.u_off);
        pm.counters = reinterpret_cast<unsigned*>(ws + wl.cnt_off);
        const hipError_t e = !mfma ? launch_attend_stream(pm, s)
                             : wide ? launch_attend_mfma32(pm, s) : launch_attend_mfma(pm, s);
        return hip_status(e, "attend_window (fused) launch");
      }
    }
  }
  p.k_win = k_win;
  p.v_win = v_win;
  p.W = W;
  return hip_status(launch_attend_valu(p, s), "attend_window launch");
}

kvq_status kvq_attend_variant(const float* q, const uint8_t* k_codes, const float* k_scales,
                              const uint8_t* v_codes, const float* v_scales, int B, int Hq,
                              int Hkv, int R, int N, int D, int bits, int group, float sm_scale,
                              int num_splits, void* workspace, size_t workspace_bytes,
                              float* out, int variant, void* stream) {
  return kvq_attend_cache(q, k_codes, k_scales, v_codes, v_scales, B, Hq, Hkv, R, N, N, D, bits,
                          group, sm_scale, num_splits, workspace, workspace_bytes, out, variant, 0,
                          stream);
}

kvq_status kvq_attend(const float* q, const uint8_t* k_codes, const float* k_scales,
                      const uint8_t* v_codes, const float* v_scales, int B, int Hq, int Hkv,
                      int R, int N, int D, int bits, int group, float sm_scale, int num_splits,
                      void* workspace, size_t workspace_bytes, float* out, void* stream) {
  return kvq_attend_variant(q, k_codes, k_scales, v_codes, v_scales, B, Hq, Hkv, R, N, D, bits,
                            group, sm_scale, num_splits, workspace, workspace_bytes, out,
                            KVQ_VARIANT_AUTO, stream);
}

kvq_status kvq_attend_noalloc(const float* q, const uint8_t* k_codes, const float* k_scales,
                              const uint8_t* v_codes, const float* v_scales, int B, int Hq,
                              int Hkv, int R, int N, int D, int bits, int group, float sm_scale,
                              int num_splits, float* out, void* stream) {
  int dev = 0;
  void* ws = nullptr;
  kvq_status st = scratch_address(&dev, &ws);
  if (st != KVQ_OK) return st;
  // The same checks as kvq_attend with the scratch as its workspace: a call
  // whose splits need more than the scratch holds fails with
  // KVQ_ERR_WORKSPACE before anything is enqueued.
  AttendProblem p;
  st = check_attend(q, k_codes, k_scales, v_codes, v_scales, B, Hq, Hkv, R, N, N, D, bits, group,
                    sm_scale, num_splits, ws, kScratchBytes, out, &p);
  if (st != KVQ_OK) {
    if (st == KVQ_ERR_WORKSPACE)
      return fail(KVQ_ERR_WORKSPACE,
                  "kvq_attend_noalloc: the call needs %zu workspace bytes, the library's "
                  "scratch holds %zu (use kvq_attend with a caller workspace, or fewer splits)",
                  kvq_attend_workspace_bytes(B, Hq, Hkv, R, N, D, num_splits), kScratchBytes);
    return st;
  }
  // Counters of this call that an earlier call with fewer (batch, KV head)
  // pairs overwrote with its partials: zero them first, on the same stream.
  const size_t counters = static_cast<size_t>(256) * B * Hkv;
  const size_t from = scratch_claim(dev, counters);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (from < counters) {
    const size_t n = counters - from;
    const size_t blocks = (n + 255) / 256;
    const unsigned grid = static_cast<unsigned>(blocks < 1024 ? blocks : 1024);
    hipLaunchKernelGGL(zero_bytes_kernel, dim3(grid), dim3(256), 0, s,
                       static_cast<unsigned char*>(ws) + from, n);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
      return fail(KVQ_ERR_HIP, "scratch clear launch: %s", hipGetErrorString(e));
  }
  return kvq_attend(q, k_codes, k_scales, v_codes, v_scales, B, Hq, Hkv, R, N, D, bits, group,
                    sm_scale, num_splits, ws, kScratchBytes, out, stream);
}

kvq_status kvq_attend_f32(const float* q, const float* k, const float* v, int B, int Hq, int Hkv,
                          int R, int N, int D, float sm_scale, int num_splits, void* workspace,
                          size_t workspace_bytes, float* out, void* stream) {
  AttendProblem p;
  kvq_status st = check_attend(q, k, nullptr, v, nullptr, B, Hq, Hkv, R, N, N, D, 32, 1, sm_scale,
                               num_splits, workspace, workspace_bytes, out, &p);
  if (st != KVQ_OK) return st;
  return hip_status(launch_attend_valu(p, static_cast<hipStream_t>(stream)),
                    "attend_f32 launch");
}

kvq_status kvq_stream_read(const void* data, size_t bytes, void* sink, void* stream) {
  if (!data || !sink) return fail(KVQ_ERR_INVALID, "null pointer argument");
  if (bytes == 0 || bytes % 16 != 0)
    return fail(KVQ_ERR_INVALID, "bytes must be a positive multiple of 16 (got %zu)", bytes);
  if (!aligned(data, 16) || !aligned(sink, 4))
    return fail(KVQ_ERR_INVALID, "data must be 16-byte aligned and sink 4-byte aligned");
  return hip_status(launch_stream_read(data, static_cast<long long>(bytes),
                                       static_cast<unsigned*>(sink),
                                       static_cast<hipStream_t>(stream)),
                    "stream_read launch");
}

const char* kvq_status_string(int status) {
  switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_INVALID: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVQ_ERR_HIP: return "HIP runtime error";
    case KVQ_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

const char* kvq_last_error(void) { return g_last_error; }

int kvq_abi_version(void) { return 10; }

kvq_status kvq_phase_trace_fetch(int kernel, void* host, size_t bytes) {
  if (host == nullptr || bytes == 0 || bytes % 8 != 0)
    return fail(KVQ_ERR_INVALID, "phase records: null host buffer or size %zu not a positive "
                "multiple of 8", bytes);
  if (kernel < 0 || kernel > 2)
    return fail(KVQ_ERR_INVALID,
                "phase records: kernel %d is not 0 (4-row), 1 (32-row) or 2 (streaming)", kernel);
  const int st = kernel == 0   ? kvq::phase_fetch_r4(host, bytes)
                 : kernel == 1 ? kvq::phase_fetch_r32(host, bytes)
                               : kvq::phase_fetch_stream(host, bytes);
  if (st == KVQ_ERR_UNSUPPORTED)
    return fail(KVQ_ERR_UNSUPPORTED, "phase records exist only in a KVQ_PHASE_TRACE build");
  if (st != KVQ_OK) return fail(KVQ_ERR_HIP, "phase records: copy from the device failed");
  return KVQ_OK;
}

}  // extern "C"
