// Streaming float32 attention over the packed cache for D = 128 in formats
// the matrix-core kernels do not take: 4- or 8-bit codes with a
// power-of-two group from 8 to 128, up to 8 query rows per KV head, with or
// without the causal rule, and with or without a float32 window of the most
// recent tokens (each a separate instantiation).
//
// Method: the blocked online softmax of "Block KV decoding: less workspace,
// more time" (huhohoo.com/en/docs/llm/kv-block-decode-cost), section "Do not
// average independently normalized blocks", and of "给长前缀列一张有单位的资源账本"
// (codingai-lec05.pages.dev resource-ledger), section "why FlashAttention need
// not keep the whole heat map": per query row a reference max m, an
// exponential sum z and an unnormalized value sum u relative to 2^m, both
// rescaled when the reference moves (lazily: only when a block's max passes
// it by more than kSLazy).  Waves and KV splits merge with the same rescale
// ("two stops of the online accumulation" on the same page).  The dequant
// is that of "KV分组打包：4-bit到底省了多少？" (huhohoo.com/docs/llm/kv-packed-groups):
// code c of a group with scale s stands for (c - qmax) * s, here one fused
// multiply-add c * s + fl32(-qmax * s) (within 2^-21 s of the exact
// product).  Plain float32 arithmetic throughout.
//
// Work split: one workgroup of 8 waves (4 for 8 rows) per (KV head, split),
// with the matrix-core kernels' XCD-aware mapping; wave w attends blocks
// w, w + waves, ... of its split.  Lane (n, q) = (lane >> 2, lane & 3) owns
// channel octet n (channels 8n .. 8n + 7), feature octet n (features 8n ..
// 8n + 7) and token octet q (tokens 8q .. 8q + 7 of each 32-token block).  In
// the block layout of kvq_layout.h each of these is one contiguous run of
// code bytes (32 at 4-bit, 64 at 8-bit), and the lane's K scales (8 channels
// of the token octet's group) and V scales (8 tokens of the feature octet's
// group) are two 16-byte runs each:
//   scores: the lane's partial dot products over its 8 channels, for every
//     query row, are summed over the 16 lanes of its token octet by a
//     reduce-scatter (two lane-swap halvings across the wave's 16-lane rows,
//     then a sum over the 4 lanes of the row), which leaves each lane the full
//     scores of R/4 rows for its 8 tokens;
//   softmax: on those scores only, the row max over the 4 token octets of a
//     quad; the probabilities go back to every lane (two lane-swap stages);
//   values: the lane accumulates u for its 8 features over its 8 tokens for
//     the whole split; the 4 token octets of a quad are summed once, at the
//     end.
// Streaming: each wave keeps its next block in flight in an LDS slot, copied
// from HBM by LDS-destination buffer loads (no VGPRs held in flight), in two
// parts: the K part (codes and scales) is refilled as soon as the block's K
// pieces are in registers, the V part as soon as its V pieces are, so each
// part has a whole block's time to land and only one part is held in
// registers at a time.
#include "kvq_internal.h"
#include "kvq_layout.h"
#include "kvq_mfma_common.h"

namespace kvq {
namespace {

constexpr int kSD = 128;
constexpr float kSLazy = 6.0f;  // the reference moves only past m + kSLazy

struct SHead {
  __amdgpu_buffer_rsrc_t kc, ksc, vc, vsc;
  long long kblock, vblock;  // code bytes per block
  int vcols;                 // V byte columns per token octet
  int vgroups;               // V scale groups per token
  int gshift;                // log2(group)
};

// One part (K or V) of a block, this lane's share: code pieces, then the two
// scale pieces.
template <int kBits>
constexpr int kSPart = kBits / 2 + 2;  // 16-byte pieces per lane and part
template <int kBits>
struct SPart {
  u32x4 c[kBits / 2];
  f32x4 s[2];
};

// LDS slot of one wave: part x (0 = K, 1 = V), piece j at
// slot + 1024 (x kSPart + j) + 16 lane.
template <int kBits>
constexpr int kSSlotBytes = 2 * 1024 * kSPart<kBits>;
// Slots per wave (blocks in flight).  One: a second slot (tried where it fits
// in LDS) doubles the burst of loads at the start, which delays every
// wave's first block and its query copy, and made the calls slower (4-bit
// group 8 on the 8 x 4096 cache 26.0 vs 22.3 us; 8 rows 33.2 vs 28.7 us).
template <int kBits, int kWaves>
constexpr int kSDepth = 1;

#define KVQ_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// s_waitcnt with vmcnt(x) (bits 3:0 and 15:14), expcnt and lgkmcnt at maximum.
#define KVQ_SVMCNT(x) ((((x) & 15) | (((x) >> 4) << 14)) | 0x0F70)

// Wait until at most `parts` (0 to 4) block parts (kSPart loads each) are in
// flight.
template <int kBits>
__device__ __forceinline__ void wait_parts(int parts) {
  switch (parts) {
    case 0: __builtin_amdgcn_s_waitcnt(KVQ_SVMCNT(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(KVQ_SVMCNT(kSPart<kBits>)); break;
    case 2: __builtin_amdgcn_s_waitcnt(KVQ_SVMCNT(2 * kSPart<kBits>)); break;
    case 3: __builtin_amdgcn_s_waitcnt(KVQ_SVMCNT(3 * kSPart<kBits>)); break;
    default: __builtin_amdgcn_s_waitcnt(KVQ_SVMCNT(4 * kSPart<kBits>)); break;
  }
}

// Start copying one part of a block into LDS (asynchronous, counted by
// vmcnt: kSPart loads).  codes / scales: the lane's byte offsets.
template <int kBits>
__device__ __forceinline__ void dma_part(unsigned char* part, __amdgpu_buffer_rsrc_t rc,
                                         unsigned codes, __amdgpu_buffer_rsrc_t rs,
                                         unsigned scales) {
  constexpr int kNt = 2;  // nontemporal cache policy: the cache is read once per call
#pragma unroll
  for (int i = 0; i < kBits / 2; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, KVQ_LDS(part + 1024 * i), 16, codes + 16 * i, 0,
                                             0, kNt);
#pragma unroll
  for (int i = 0; i < 2; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, KVQ_LDS(part + 1024 * (kBits / 2 + i)), 16,
                                             scales + 16 * i, 0, 0, kNt);
}

// K part of block blk: channel octet n of tokens 8q .. 8q + 7 and the scales
// of those channels in the token octet's group.
template <int kBits>
__device__ __forceinline__ void dma_k(unsigned char* slot, const SHead& h, int blk, int n, int q) {
  const unsigned co = static_cast<unsigned>(blk * h.kblock) +
                      static_cast<unsigned>((n * 4 * kBits + kBits * q) * 8);
  const int tok = blk * kBlockTokens + 8 * q;
  const unsigned so = static_cast<unsigned>(((tok >> h.gshift) * kSD + 8 * n) * 4);
  dma_part<kBits>(slot, h.kc, co, h.ksc, so);
}

// V part of block blk: feature octet n of tokens 8q .. 8q + 7 and the scales
// of those tokens in the feature octet's group.
template <int kBits>
__device__ __forceinline__ void dma_v(unsigned char* slot, const SHead& h, int blk, int n, int q) {
  const unsigned co = static_cast<unsigned>(blk * h.vblock) +
                      static_cast<unsigned>((q * h.vcols + kBits * n) * 8);
  const unsigned so = static_cast<unsigned>(
      ((blk * h.vgroups + ((8 * n) >> h.gshift)) * kBlockTokens + 8 * q) * 4);
  dma_part<kBits>(slot + 1024 * kSPart<kBits>, h.vc, co, h.vsc, so);
}

template <int kBits>
__device__ __forceinline__ void read_part(SPart<kBits>& r, const unsigned char* part, int lane) {
  const unsigned char* b = part + 16 * lane;
#pragma unroll
  for (int i = 0; i < kBits / 2; ++i) r.c[i] = *reinterpret_cast<const u32x4*>(b + 1024 * i);
#pragma unroll
  for (int i = 0; i < 2; ++i)
    r.s[i] = *reinterpret_cast<const f32x4*>(b + 1024 * (kBits / 2 + i));
}

// Codes e = 0..3 of a 4-byte word as float: its bytes (8-bit) or their low
// or high nibbles (4-bit).  The nibble mask is applied in an asm statement so
// that the compiler cannot merge it into per-code bit-field extracts: the
// masked word's bytes then convert with one v_cvt_f32_ubyteN each.
template <int kBits>
__device__ __forceinline__ void codes4(unsigned w, bool hi, float c[4]) {
  unsigned x = w;
  if (kBits == 4) {
    const unsigned y = hi ? w >> 4 : w;
    asm("v_and_b32_e32 %0, 0x0f0f0f0f, %1" : "=v"(x) : "v"(y));
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) c[e] = static_cast<float>((x >> (8 * e)) & 0xFFu);
}

// ---- cross-lane steps (lane = 4 n + q) -----------------------------------------
// Reduce-scatter halves, one swap and one add each: scatter32 gives the lanes
// below 32 (bit 5 clear) x summed with the lane 32 away and the others y
// summed likewise; scatter16 does the same across lanes 16 apart (bit 4).
__device__ __forceinline__ float scatter32(float x, float y) {
  const auto r = __builtin_amdgcn_permlane32_swap(as_u32(x), as_u32(y), false, false);
  return as_f32(r[0]) + as_f32(r[1]);
}
__device__ __forceinline__ float scatter16(float x, float y) {
  const auto r = __builtin_amdgcn_permlane16_swap(as_u32(x), as_u32(y), false, false);
  return as_f32(r[0]) + as_f32(r[1]);
}
// x summed over the 4 lanes of its DPP row with the same q (lanes 4 apart).
__device__ __forceinline__ float sum_over_n4(float x) {
  x += dpp<kRowRor8>(x);
  return x + dpp<kRowRor4>(x);
}
// Sum / max over the 4 lanes of a quad (its 4 token octets).
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E;  // quad_perm [1,0,3,2], [2,3,0,1]
__device__ __forceinline__ float quad_sum(float x) {
  x += dpp<kQuadXor1>(x);
  return x + dpp<kQuadXor2>(x);
}
__device__ __forceinline__ float quad_max(float x) {
  x = fmaxf(x, dpp<kQuadXor1>(x));
  return fmaxf(x, dpp<kQuadXor2>(x));
}
// Values of the rows held by other lanes: v[j] (row (R/2) b5 + (R/4) b4 + j,
// b5 / b4 the lane's bits 5 / 4) from every lane of the same quad position, in
// absolute row order: out[r] for r < R.
template <int kRows>
__device__ __forceinline__ void gather_rows(const float (&v)[kRows / 4], float (&out)[kRows]) {
#pragma unroll
  for (int j = 0; j < kRows / 4; ++j) {
    float lo, hi;  // the value of the lane with bit 4 clear / set
    swap16(v[j], lo, hi);
    swap32(lo, out[j], out[kRows / 2 + j]);
    swap32(hi, out[kRows / 4 + j], out[kRows / 2 + kRows / 4 + j]);
  }
}

// Query rows in LDS: qs[r][hf][n] holds channels 8n + 4hf .. 8n + 4hf + 3 of
// row r, so the 16 lanes of a token octet read 256 contiguous bytes (rows
// past `rows` are zero).
template <int kRows>
struct SQuery {
  f32x4 qs[kRows][2][16];
};

// Where a lane's query values come from: registers (up to 4 rows: 32 VGPRs)
// or the LDS copy above (8 rows), read per channel quad and block.
template <int kRows, bool kInRegs>
struct QSource;
template <int kRows>
struct QSource<kRows, true> {
  f32x4 q[kRows][2];
  __device__ __forceinline__ f32x4 get(int r, int hf) const { return q[r][hf]; }
};
template <int kRows>
struct QSource<kRows, false> {
  const SQuery<kRows>* sq;
  int n;
  __device__ __forceinline__ f32x4 get(int r, int hf) const { return sq->qs[r][hf][n]; }
};

template <int kBits, int kRows, int kWaves>
struct SSmem {
  // up to 4 rows: each wave's own copy of the query rows, as SQuery
  f32x4 wq[kRows <= 4 ? kWaves : 1][kRows <= 4 ? kRows * 32 : 1];
  union {
    unsigned char ring[kWaves][kSDepth<kBits, kWaves>][kSSlotBytes<kBits>];  // block slots
    float wu[kWaves][kRows][kSD];                     // the merge (after the loop)
    WinSmem<kRows> win;                               // a recent-token window part
  } u;
  SQuery<kRows> q;
  float wm[kWaves][kRows];
  float wz[kWaves][kRows];
  int last;
};

// Scores of the lane's token octet in one block.  Each lane first forms its
// partial dot products over its 8 channels for every row and token; a
// reduce-scatter then leaves it the full scores of R/4 rows: out[j][t] is
// row (R/2) b5 + (R/4) b4 + j, token 8q + t (b5 / b4: lane bits 5 / 4; the
// 4 lanes of a DPP row with the same q hold the same values).
// qscale: sm_scale * log2 e, folded into the K scales (scores in base-2 units).
template <int kBits, int kRows, typename QS>
__device__ __forceinline__ void block_scores(const SPart<kBits>& kp, const QS& qsrc,
                                             float qscale, float (&out)[kRows / 4][8]) {
  float s[kRows][8];
  constexpr float kQmax = kBits == 4 ? 7.0f : 127.0f;
#pragma unroll
  for (int r = 0; r < kRows; ++r)
#pragma unroll
    for (int t = 0; t < 8; ++t) s[r][t] = 0.0f;
  // channel quad hf = channels 8n + 4hf .. 8n + 4hf + 3; its codes sit in
  // dword 2j + hf: token pair j (low nibbles token 2j, high 2j + 1) at 4-bit,
  // token j at 8-bit.
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    f32x4 qh[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) qh[r] = qsrc.get(r, hf);
    float ks[4], kb[4];  // K scale times qscale, and -qmax times that
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ks[e] = kp.s[hf][e] * qscale;
      kb[e] = -kQmax * ks[e];
    }
#pragma unroll
    for (int j = 0; j < kBits; ++j) {
      const int d = 2 * j + hf;
      const unsigned w = kp.c[d / 4][d % 4];
#pragma unroll
      for (int part = 0; part < (kBits == 4 ? 2 : 1); ++part) {
        const int t = kBits == 4 ? 2 * j + part : j;
        float c[4];
        codes4<kBits>(w, part == 1, c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float kv = fmaf(c[e], ks[e], kb[e]);  // (c - qmax) s qscale
#pragma unroll
          for (int r = 0; r < kRows; ++r) s[r][t] = fmaf(qh[r][e], kv, s[r][t]);
        }
      }
    }
  }
  // Reduce over the 16 lanes of each token octet (lanes 4 apart): halve the
  // rows across lane bit 5, then bit 4, then sum over the 4 lanes in the row.
  float h[kRows / 2][8];
#pragma unroll
  for (int r = 0; r < kRows / 2; ++r)
#pragma unroll
    for (int t = 0; t < 8; ++t) h[r][t] = scatter32(s[r][t], s[r + kRows / 2][t]);
#pragma unroll
  for (int j = 0; j < kRows / 4; ++j)
#pragma unroll
    for (int t = 0; t < 8; ++t) out[j][t] = sum_over_n4(scatter16(h[j][t], h[j + kRows / 4][t]));
}

// The lazy online-softmax update for one block on the lane's R/4 rows (as
// block_scores leaves them); s becomes p = 2^(s - m).  m, z: the lane's rows
// (z over its token octet only); u: every row.  ntok: how many of the lane's
// 8 tokens are in the split (the rest, past the cache's end, take no part).
// kCausal: nrow[j] more bounds row j's tokens (its query's position), and a
// row that has seen no legal key yet keeps m = -inf, its exponents taken
// against 0 (so (-inf) - (-inf) is never formed) and z = u = 0.
// Every lane of the wave calls it.
template <int kRows, bool kCausal>
__device__ __forceinline__ void block_softmax(float (&s)[kRows / 4][8], int ntok,
                                              const int (&nrow)[kRows / 4],
                                              float (&m)[kRows / 4], float (&z)[kRows / 4],
                                              float (&u)[kRows][8], bool& live) {
  constexpr int kL = kRows / 4;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const bool ok = t < ntok;
#pragma unroll
    for (int j = 0; j < kL; ++j)
      s[j][t] = ok && (!kCausal || t < nrow[j]) ? s[j][t] : -INFINITY;
  }
  float bm[kL];
  bool up = false;
#pragma unroll
  for (int j = 0; j < kL; ++j) {
    float x = s[j][0];
#pragma unroll
    for (int t = 1; t < 8; ++t) x = fmaxf(x, s[j][t]);
    bm[j] = quad_max(x);  // the block's max of the row (all 32 tokens)
    up = up || bm[j] > m[j] + kSLazy;
  }
  if (!live || __builtin_amdgcn_ballot_w64(up) != 0) {  // wave-uniform
    float a[kL];
#pragma unroll
    for (int j = 0; j < kL; ++j) {
      const float mn = live ? (bm[j] > m[j] + kSLazy ? bm[j] : m[j]) : bm[j];
      a[j] = live && (!kCausal || m[j] != -INFINITY) ? fast_exp2(m[j] - mn) : 0.0f;
      z[j] *= a[j];
      m[j] = mn;
    }
    float ar[kRows];
    gather_rows<kRows>(a, ar);
#pragma unroll
    for (int r = 0; r < kRows; ++r)
#pragma unroll
      for (int f = 0; f < 8; ++f) u[r][f] *= ar[r];
    live = true;
  }
#pragma unroll
  for (int j = 0; j < kL; ++j) {
    const float ref = kCausal && m[j] == -INFINITY ? 0.0f : m[j];
    float zs = 0.0f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      s[j][t] = fast_exp2(s[j][t] - ref);
      zs += s[j][t];
    }
    z[j] += zs;
  }
}

// u[r][f] += sum over the lane's tokens t of p[r][t] (c - qmax) sV, feature
// 8n + f.  4-bit: dword 2j + hh holds tokens 4hh .. 4hh + 3 of features 2j
// (low nibbles) and 2j + 1 (high); 8-bit: dword 2f + hh holds them for
// feature f.
template <int kBits, int kRows>
__device__ __forceinline__ void block_values(const SPart<kBits>& vp, const float (&p)[kRows][8],
                                             float (&u)[kRows][8]) {
  constexpr float kQmax = kBits == 4 ? 7.0f : 127.0f;
  float vs[8], vb[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    vs[e] = vp.s[0][e];
    vs[e + 4] = vp.s[1][e];
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) vb[t] = -kQmax * vs[t];
#pragma unroll
  for (int d = 0; d < 2 * kBits; ++d) {
    const unsigned w = vp.c[d / 4][d % 4];
    const int hh = d & 1;
#pragma unroll
    for (int part = 0; part < (kBits == 4 ? 2 : 1); ++part) {
      const int f = kBits == 4 ? 2 * (d >> 1) + part : d >> 1;
      float c[4];
      codes4<kBits>(w, part == 1, c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 4 * hh + e;
        const float vv = fmaf(c[e], vs[t], vb[t]);  // (c - qmax) s
#pragma unroll
        for (int r = 0; r < kRows; ++r) u[r][f] = fmaf(p[r][t], vv, u[r][f]);
      }
    }
  }
}

// kCausal: a causal chunk (row r is query r % R at position pos_end - R +
// r % R and reads tokens up to its own); only tokens past pos_end - R can be
// masked, and a row with no legal key in the split returns m = -inf, z = 0.
// kWindow: the last p.win_parts splits of each head are parts of a float32
// window of the most recent tokens (window_part, kvq_mfma_common.h), placed
// after every head's packed splits in the grid (wg_slot).
template <int kBits, int kRows, int kWaves, bool kCausal, bool kWindow>
__global__ __launch_bounds__(kWaves * 64) void attend_stream_kernel(AttendProblem p) {
  constexpr int kThreads = kWaves * 64;
  // Outputs per thread in the merge and the split combine: row r, features
  // f0 .. f0 + kF - 1 (threads past the kRows rows take no part).
  constexpr int kF = (kRows * kSD + kThreads - 1) / kThreads;
  static_assert(kSD % kF == 0, "whole rows per thread group");
  __shared__ SSmem<kBits, kRows, kWaves> sm;
  phase_mark(kMarkStart);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane >> 2;  // channel / feature octet
  const int q = lane & 3;   // token octet

  const int heads = p.B * p.Hkv;
  const WgSlot wslot = wg_slot(blockIdx.x, heads, p.splits, kWindow ? p.win_parts : 0);
  const int head = wslot.head, split = wslot.split;
  const long long bh = head;
  const int rows = p.rows;
  if (kWindow && split >= p.splits - p.win_parts) {  // a window part (the whole workgroup)
    const int r = tid * kF / kSD, f0 = (tid * kF) % kSD;
    float U[kF], M, Z;
    window_part<kRows, kThreads, kF, kF, 0>(p, sm.u.win, bh, split - (p.splits - p.win_parts),
                                            r, f0, U, M, Z);
    split_combine<kF, kF, 0>(p, split, bh, r, f0, U, M, Z, &sm.last);
    return;
  }
  const Layout lay = make_layout(p.cap, kSD, kBits, p.group);
  SHead h;
  h.kblock = lay.kblock_bytes;
  h.vblock = lay.vblock_bytes;
  h.vcols = lay.vcols;
  h.vgroups = lay.vgroups;
  h.gshift = __builtin_ctz(p.group);
  h.kc = head_rsrc(p.k_codes + bh * k_code_bytes_per_head(lay), k_code_bytes_per_head(lay));
  h.ksc = head_rsrc(p.k_scales + bh * k_scales_per_head(lay), k_scales_per_head(lay) * 4);
  h.vc = head_rsrc(p.v_codes + bh * v_code_bytes_per_head(lay), v_code_bytes_per_head(lay));
  h.vsc = head_rsrc(p.v_scales + bh * v_scales_per_head(lay), v_scales_per_head(lay) * 4);

  const int t_begin = split * p.tokens_per_split;
  const int t_end = min(p.N, t_begin + p.tokens_per_split);
  const int b_begin = t_begin / kBlockTokens;
  const int b_end = t_end > t_begin ? (t_end + kBlockTokens - 1) / kBlockTokens : b_begin;
  const int b_first = b_begin + wave;
  const int cnt = b_first < b_end ? (b_end - 1 - b_first) / kWaves + 1 : 0;  // wave-uniform

  // The query rows (a descriptor over the head's `rows` rows reads zeros past
  // them).  Up to 4 rows each wave copies them into its own LDS area with
  // LDS-destination loads issued ahead of its first blocks, then reads its
  // lanes' values into registers: no register is loaded from memory before
  // the loop, which would make the compiler wait for every block copy in
  // flight at the loop's entry.  For 8 rows they stay in LDS (stored before
  // any block copy is in flight, since an LDS store is ordered after every
  // LDS-destination load issued before it) and are read per block.
  constexpr bool kQRegs = kRows <= 4;
  const __amdgpu_buffer_rsrc_t qrs = head_rsrc(p.q + bh * rows * kSD, rows * kSD * 4);
  QSource<kRows, kQRegs> qsrc;
  constexpr int kDepth = kSDepth<kBits, kWaves>;
  if constexpr (kQRegs) {
    // piece i = (r * 2 + hf) * 16 + o of the copy holds channels 8o + 4hf ..
    // 8o + 4hf + 3 of row r; lane ell of copy step c loads piece 64 c + ell
#pragma unroll
    for (int c = 0; c < kRows * 32 / 64; ++c) {
      const int i = 64 * c + lane, r = i >> 5, hf = (i >> 4) & 1, o = i & 15;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          qrs, KVQ_LDS(&sm.wq[wave][64 * c]), 16,
          static_cast<unsigned>((r * kSD + 8 * o + 4 * hf) * 4), 0, 0, 0);
    }
  } else {
    static_assert(kRows * 32 <= kThreads, "one query piece per thread");
    const int qr = tid >> 5, qhf = (tid >> 4) & 1, qo = tid & 15;
    if (qr < kRows)
      sm.q.qs[qr][qhf][qo] =
          buf_f4(qrs, static_cast<unsigned>((qr * kSD + 8 * qo + 4 * qhf) * 4), 0);
    __syncthreads();
    qsrc.sq = &sm.q;
    qsrc.n = n;
  }
  // Block i of the wave sits in slot i % kDepth; the first kDepth blocks go
  // out at once, in the order K(0) V(0) K(1) V(1) ...
#pragma unroll
  for (int d = 0; d < kDepth; ++d) {
    if (d < cnt) {
      dma_k<kBits>(sm.u.ring[wave][d], h, b_first + d * kWaves, n, q);
      dma_v<kBits>(sm.u.ring[wave][d], h, b_first + d * kWaves, n, q);
    }
  }
  if constexpr (kQRegs) {
    wait_parts<kBits>(2 * min(kDepth, cnt));  // the query copy has landed
#pragma unroll
    for (int r = 0; r < kRows; ++r)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) qsrc.q[r][hf] = sm.wq[wave][(r * 2 + hf) * 16 + n];
  }
  phase_mark(kMarkQReady);

  // m, z: the lane's R/4 rows (row (R/2) b5 + (R/4) b4 + j); u: every row,
  // features 8n .. 8n + 7, over the lane's token octet.
  constexpr int kL = kRows / 4;
  float m[kL], z[kL], u[kRows][8];
#pragma unroll
  for (int j = 0; j < kL; ++j) {
    m[j] = -INFINITY;
    z[j] = 0.0f;
  }
#pragma unroll
  for (int r = 0; r < kRows; ++r)
#pragma unroll
    for (int f = 0; f < 8; ++f) u[r][f] = 0.0f;
  bool live = false;
  // Causal limit of the lane's rows (R/2) b5 + (R/4) b4 + j: the last token
  // each may read.
  int lim[kL];
  {
    const int r0 = (kRows / 2) * (lane >> 5) + (kRows / 4) * ((lane >> 4) & 1);
#pragma unroll
    for (int j = 0; j < kL; ++j) lim[j] = kCausal ? p.pos_end - p.R + (r0 + j) % p.R : 0;
  }

  // Parts are issued in the order K(0) V(0) K(1) V(1) ...: K(i + kDepth) once
  // K(i) is in registers, V(i + kDepth) once V(i) is.  So K(i) has landed
  // once no more than the parts issued after it (V(i), then K and V of the
  // blocks up to i + kDepth - 1) are pending, and V(i) once no more than the
  // parts after it (K and V up to block i + kDepth - 1, then K(i + kDepth)).
  for (int i = 0; i < cnt; ++i) {
    const int blk = b_first + i * kWaves;
    unsigned char* slot = sm.u.ring[wave][i % kDepth];
    const int ahead = min(kDepth - 1, cnt - 1 - i);  // blocks already issued past i
    const bool more = i + kDepth < cnt;              // block i + kDepth exists
    priority_by_blocks_left(i, cnt);  // waves that share a SIMD finish together
    float s[kL][8];
    {
      wait_parts<kBits>(1 + 2 * ahead);  // K(i) in the slot
      if (i == 0) phase_mark(kMarkFirstBlock);
      SPart<kBits> kp;
      read_part<kBits>(kp, slot, lane);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the K part has been read
      if (more) dma_k<kBits>(slot, h, blk + kDepth * kWaves, n, q);
      block_scores<kBits, kRows>(kp, qsrc, p.qscale, s);
    }
    {
      const int tok0 = blk * kBlockTokens + 8 * q;
      int nrow[kL];
#pragma unroll
      for (int j = 0; j < kL; ++j) nrow[j] = lim[j] - tok0 + 1;
      block_softmax<kRows, kCausal>(s, t_end - tok0, nrow, m, z, u, live);
    }
    {
      wait_parts<kBits>(2 * ahead + (more ? 1 : 0));  // V(i) in the slot
      SPart<kBits> vp;
      read_part<kBits>(vp, slot + 1024 * kSPart<kBits>, lane);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the V part has been read
      if (more) dma_v<kBits>(slot, h, blk + kDepth * kWaves, n, q);
      float pr[kRows][8];  // p of every row for the lane's tokens
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        float pj[kL], pa[kRows];
#pragma unroll
        for (int j = 0; j < kL; ++j) pj[j] = s[j][t];
        gather_rows<kRows>(pj, pa);
#pragma unroll
        for (int r = 0; r < kRows; ++r) pr[r][t] = pa[r];
      }
      block_values<kBits, kRows>(vp, pr, u);
    }
  }

  __builtin_amdgcn_s_setprio(0);
  phase_mark(kMarkLoopEnd);

  // ---- merge: the 4 token octets, then the waves through LDS ---------------
#pragma unroll
  for (int j = 0; j < kL; ++j) z[j] = quad_sum(z[j]);
#pragma unroll
  for (int r = 0; r < kRows; ++r)
#pragma unroll
    for (int f = 0; f < 8; ++f) u[r][f] = quad_sum(u[r][f]);
  __syncthreads();  // every wave is done with its slot (aliased by the merge area)
  if (q == 0) {
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      f32x4 a, b;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[e] = u[r][e];
        b[e] = u[r][e + 4];
      }
      *reinterpret_cast<f32x4*>(&sm.u.wu[wave][r][8 * n]) = a;
      *reinterpret_cast<f32x4*>(&sm.u.wu[wave][r][8 * n + 4]) = b;
    }
  }
  if ((lane & 15) == 0) {  // one lane per (bit 5, bit 4): rows (R/2) b5 + (R/4) b4 + j
    const int r0 = (kRows / 2) * (lane >> 5) + (kRows / 4) * ((lane >> 4) & 1);
#pragma unroll
    for (int j = 0; j < kL; ++j) {
      sm.wm[wave][r0 + j] = m[j];
      sm.wz[wave][r0 + j] = z[j];
    }
  }
  __syncthreads();
  // outputs per thread: row r, features f0 .. f0 + kF - 1
  const int r = tid * kF / kSD;
  const int f0 = (tid * kF) % kSD;
  const int rr = r < kRows ? r : kRows - 1;  // in-range row for the LDS reads
  float M = -INFINITY, Z = 0.0f, U[kF];
#pragma unroll
  for (int j = 0; j < kF; ++j) U[j] = 0.0f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.wm[w][rr]);
  if (M != -INFINITY) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm.wm[w][rr];
      if (mw == -INFINITY) continue;
      const float x = fast_exp2(mw - M);
      Z = fmaf(x, sm.wz[w][rr], Z);
#pragma unroll
      for (int j = 0; j < kF; ++j) U[j] = fmaf(x, sm.u.wu[w][rr][f0 + j], U[j]);
    }
  }
  phase_mark(kMarkMerged);
  if (p.splits == 1) {
    if (r < rows) {
#pragma unroll
      for (int j = 0; j < kF; ++j)  // causal: Z = 0 for a row with no legal key
        p.out[(bh * rows + r) * kSD + f0 + j] = !kCausal || Z > 0.0f ? U[j] / Z : 0.0f;
    }
    phase_mark(kMarkEnd);
    return;
  }
  split_combine<kF, kF, 0>(p, split, bh, r, f0, U, M, Z, &sm.last);
  phase_mark(kMarkEnd);
}

#undef KVQ_SVMCNT

}  // namespace

int phase_fetch_stream(void* host, size_t bytes) { return phase_fetch(host, bytes); }

// Waves per workgroup: 8 up to 4 rows (138-144 VGPRs), 4 for 8 rows (222-225
// VGPRs, two workgroups per compute unit).  The automatic split count aims at
// two waves per SIMD either way.  (8 waves for 8 rows measured the same at
// the automatic split count; 12 waves up to 4 rows were slower.)
static constexpr int waves_for(int rows) { return rows <= 4 ? 8 : 4; }

int stream_waves(int bits, int rows) {
  (void)bits;
  return waves_for(rows > 4 ? 8 : 4);
}

template <int kBits, int kRows>
static hipError_t launch_stream(const AttendProblem& p, hipStream_t stream) {
  constexpr int kWaves = waves_for(kRows);
  const unsigned grid = static_cast<unsigned>(p.splits) * p.B * p.Hkv;
  if (p.win_parts > 0) {
    if (p.causal)
      hipLaunchKernelGGL((attend_stream_kernel<kBits, kRows, kWaves, true, true>), dim3(grid),
                         dim3(kWaves * 64), 0, stream, p);
    else
      hipLaunchKernelGGL((attend_stream_kernel<kBits, kRows, kWaves, false, true>), dim3(grid),
                         dim3(kWaves * 64), 0, stream, p);
  } else if (p.causal) {
    hipLaunchKernelGGL((attend_stream_kernel<kBits, kRows, kWaves, true, false>), dim3(grid),
                       dim3(kWaves * 64), 0, stream, p);
  } else {
    hipLaunchKernelGGL((attend_stream_kernel<kBits, kRows, kWaves, false, false>), dim3(grid),
                       dim3(kWaves * 64), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_attend_stream(const AttendProblem& p, hipStream_t stream) {
  const bool r8 = p.rows > 4;
  if (p.bits == 8) return r8 ? launch_stream<8, 8>(p, stream) : launch_stream<8, 4>(p, stream);
  return r8 ? launch_stream<4, 8>(p, stream) : launch_stream<4, 4>(p, stream);
}

}  // namespace kvq
