// Matrix-core fused attention for the 4- or 8-bit, group-32, D=128 packed
// cache with 5 to 32 query rows per KV head (GQA group x queries), rows
// padded to 16 or 32 so both products fill whole 16x16 matrix-core tiles.
//
// Method: the blocked online softmax of "Block KV decoding: less workspace,
// more time" (huhohoo.com/en/docs/llm/kv-block-decode-cost), section "Do not
// average independently normalized blocks", and of "给长前缀列一张有单位的资源账本"
// (codingai-lec05.pages.dev resource-ledger), section "why FlashAttention need
// not keep the whole heat map": per query row a reference max m, an
// exponential sum z and an unnormalized value sum u relative to 2^m, both
// rescaled by 2^(m_old - m_new) when the reference moves (lazily: only when a
// block's max exceeds it by more than 2^kLazy, which bounds p = 2^(s - m)).
// Waves and KV splits are merged with the same rescale ("two stops of the
// online accumulation" on the same page).
//
// Packed format: the 32-token block byte order of kvq_layout.h, whose K and V
// blocks hand each lane its matrix-core operand bytes at consecutive
// addresses (see the 4-row kernel in kvq_attend_mfma.hip for the byte map).
// Codes become exact fp16 (c - 7) operands; float32 factors are split into
// fp16 hi + lo (kvq_mfma_common.h).
//
// Math per 32-token block, one wave, row tile t = 0, 1 (rows 16t .. 16t+15):
//   S^T[pair][16t + n] = codes^T (A: 16 token pairs x 32 channels, low and
//     high nibbles as two products) x q~^T (B: 32 channels x 16 rows), with
//     the hi and lo halves of q~ accumulated into the same tile;
//   u[16t + m][f] += p~_g (A: 16 rows x 32 tokens, p~ = p * sV[token][g])
//     x V codes (B: 32 tokens x 16 feature pairs of value group g).
// The score tile gives lane (n, q) rows 16t + n and tokens 8q .. 8q+7, which
// is exactly the A operand of the value product: no data moves between the
// two products.
//
// q~ = q * qscale * sK[d][G] is formed per block: q * qscale sits in LDS,
// prescaled per row by a power of two that puts its largest element in
// [2^9, 2^10); K scales below 32 then keep every q~ inside the fp16 range
// (a block whose K scales reach 32 is rescaled by a power of two first).
#include "kvq_internal.h"
#include "kvq_layout.h"
#include "kvq_mfma_common.h"

namespace kvq {
namespace {

constexpr int kW = 4;            // waves per workgroup
constexpr int kT = kW * 64;      // threads per workgroup
constexpr int kR = 32;           // query rows per KV head (padded)
constexpr int kD = 128;
template <int kBits>
constexpr int kBB = 512 * kBits; // K or V code bytes of one 32-token block
template <int kBits>
constexpr int kKStep = 128 * kBits;  // lane code bytes: K k-step stride
template <int kBits>
constexpr int kVStep = 32 * kBits;   //   and V value-group stride
constexpr int kBS = 128;         // K or V scales of one block
constexpr int kQStride = 132;    // LDS row of q: 4 words of padding keep the
                                 // 16 rows read by a quarter-wave on distinct banks
constexpr float kLazy = 6.0f;    // reference moves only past m + kLazy
constexpr int kSvTop = 9;        // V prescale: max V scale * 2^Sv in [2^8, 2^9),
constexpr int kSvLow = 2;        //   kept while it stays in [2^2, 2^9)
constexpr int kQTop = 10;        // q rows prescaled to max |.| in [2^9, 2^10)
constexpr float kSkMax = 32.0f;  // K scales below this need no block rescale

struct alignas(16) Smem32 {
  union {
    float qs[kR][kQStride];      // q * qscale * 2^Sq(row)
    float wu[2][kR][kD];         // u of two waves at a time, for the merge
    WinSmem<kR> win;             // a recent-token window part
  } u;
  float sks[kW][kBS];            // this block's K scales (per wave), channel order
  float svs[kW][kBS];            // this block's V scales (per wave), [group][token]
  float alp[kW][kR];             // rescale factors of a reference move (per wave)
  float qus[kR];                 // 2^-Sq(row)
  float wm[kW][kR];
  float wz[kW][kR];
  int last;
};

template <int kBits>
struct Regs32 {
  typename CodeOps<kBits>::words k[4];  // K codes, k-step 0..3
  typename CodeOps<kBits>::words v[4];  // V codes, value group 0..3
  float2 ks;    // K scales 2 lane, 2 lane + 1 of the block
  float2 vs;    // V scales 2 lane, 2 lane + 1 of the block ([group][token])
};

// Buffer descriptors of one KV head's four arrays (kvq_mfma_common.h): the
// block offset rides in an SGPR, the lane offset in a VGPR.
struct Head32 {
  __amdgpu_buffer_rsrc_t kc, ksc, vc, vsc;
};

struct Lanes32 {
  unsigned k_off, v_off, s_off;  // byte offsets of this lane in a block
};

template <int kBits>
__device__ __forceinline__ void load_scales32(Regs32<kBits>& r, const Head32& h, int blk,
                                              const Lanes32& o) {
  r.ks = buf_f2(h.ksc, o.s_off, blk * kBS * 4);
  r.vs = buf_f2(h.vsc, o.s_off, blk * kBS * 4);
}
template <int kBits>
__device__ __forceinline__ void load_block32(Regs32<kBits>& r, const Head32& h, int blk,
                                             const Lanes32& o) {
  load_scales32(r, h, blk, o);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r.k[i] = CodeOps<kBits>::load(h.kc, o.k_off + i * kKStep<kBits>, blk * kBB<kBits>);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r.v[i] = CodeOps<kBits>::load(h.vc, o.v_off + i * kVStep<kBits>, blk * kBB<kBits>);
}

// Running state of one wave.  Lane (n, q) owns score rows 16t + n (t = 0, 1):
// m[t] is that row's reference max (equal in all its lanes), z[t] the sum of
// p over this lane's tokens 8q .. 8q+7 of every block (summed over the four
// q-blocks at the end).  acc[g][t][e] holds u of rows 16t + 4q + i, features
// 32g + 2n + e, in units of 2^(m + sv).  vscale = 2^sv multiplies the V
// scales parked in LDS; vhi / vlo bound the V scales that keep sv valid.
struct State32 {
  float m[2], z[2];
  f32x4 acc[4][2][2];
  int sv;
  float vscale, vhi, vlo;
  bool live;
};

// fp16 hi/lo operands of the 8 products x[j] = a[j] * b[j], j in k-slot
// order: hi = fp16(fp16(a) * fp16(b)) (one packed multiply per pair), lo =
// the residual x - hi, from one fused multiply-add per value rounded once to
// fp16 (v_fma_mixlo_f16 / v_fma_mixhi_f16 widen the fp16 hi internally).
// a, b are float32 with their fp16 (round-toward-zero) pairs a16, b16
// precomputed in the same order.  The eight mix instructions are one asm
// statement with early-clobber outputs (no output shares a register with an
// input), ending with s_nop 1: the compiler's hazard tracking does not see
// inside inline asm, and a matrix-core instruction reading a VGPR that a
// VALU instruction just wrote needs two wait states.
__device__ __forceinline__ void product_hilo(const float a[8], const float b[8],
                                             const half2_t a16[4], const half2_t b16[4],
                                             half8_t& hi, half8_t& lo) {
  u32x4 h, l;
#pragma unroll
  for (int i = 0; i < 4; ++i) h[i] = __builtin_bit_cast(unsigned, a16[i] * b16[i]);
  unsigned l0, l1, l2, l3;
  asm("v_fma_mixlo_f16 %0, %4, %5, -%20 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %0, %6, %7, -%20 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixlo_f16 %1, %8, %9, -%21 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %1, %10, %11, -%21 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixlo_f16 %2, %12, %13, -%22 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %2, %14, %15, -%22 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixlo_f16 %3, %16, %17, -%23 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %3, %18, %19, -%23 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
      "s_nop 1"
      : "=&v"(l0), "=&v"(l1), "=&v"(l2), "=&v"(l3)
      : "v"(a[0]), "v"(b[0]), "v"(a[1]), "v"(b[1]), "v"(a[2]), "v"(b[2]), "v"(a[3]), "v"(b[3]),
        "v"(a[4]), "v"(b[4]), "v"(a[5]), "v"(b[5]), "v"(a[6]), "v"(b[6]), "v"(a[7]), "v"(b[7]),
        "v"(h[0]), "v"(h[1]), "v"(h[2]), "v"(h[3]));
  l[0] = l0;
  l[1] = l1;
  l[2] = l2;
  l[3] = l3;
  hi = __builtin_bit_cast(half8_t, h);
  lo = __builtin_bit_cast(half8_t, l);
}

__device__ __forceinline__ half2_t pk16(float x, float y) {
  return __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(x, y));
}

// kMasked: mask tokens >= t_end; kCausal (implies kMasked): also mask, for
// score row 16t + n, the tokens after its query's position lim[t], and keep
// rows that have seen no legal key at m = -inf (exponents then taken
// against 0, so (-inf) - (-inf) is never formed).
template <int kBits, int kTiles, bool kMasked, bool kCausal>
__device__ __forceinline__ void attend_block32(Smem32& sm, Regs32<kBits>& br, int tok0, int t_end,
                                               const typename CodeOps<kBits>::consts& cc,
                                               State32& st,
                                               const Head32& h, int next, const Lanes32& lo,
                                               const float us_row[2], const float (&qk)[2][4][8],
                                               const int (&lim)[2]) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;
  const int q = lane >> 4;

  // ---- block set-up: scale guards, then this block's scales into LDS ------
  const float lks = fmaxf(br.ks.x, br.ks.y);
  const float lvs = fmaxf(br.vs.x, br.vs.y);
  // A block whose K scales reach kSkMax is scaled down by 2^-e (kf) and its
  // scores back up (kun); otherwise both are 1.
  float kf = 1.0f, kun = 1.0f;
  if (__builtin_amdgcn_ballot_w64(lks >= kSkMax) != 0) {
    float mx = fmaxf(lks, dpp<kRowRor1>(lks));
    mx = fmaxf(mx, dpp<kRowRor2>(mx));
    mx = fmaxf(mx, dpp<kRowRor4>(mx));
    mx = fmaxf(mx, dpp<kRowRor8>(mx));
    mx = qblock_max(mx);
    const int e = __builtin_amdgcn_frexp_expf(mx);
    kf = __builtin_ldexpf(1.0f, -e);
    kun = __builtin_ldexpf(1.0f, e);
  }
  // V prescale 2^sv: set so the largest V scale lands in [2^8, 2^9), moved
  // only when the block's largest V scale leaves [2^kSvLow, 2^kSvTop) after
  // scaling (u is rescaled by the change; z does not carry it).
  if (!st.live || __builtin_amdgcn_ballot_w64(!(lvs < st.vhi)) != 0 ||
      __builtin_amdgcn_ballot_w64(lvs >= st.vlo) == 0) {
    float vmx = fmaxf(lvs, dpp<kRowRor1>(lvs));
    vmx = fmaxf(vmx, dpp<kRowRor2>(vmx));
    vmx = fmaxf(vmx, dpp<kRowRor4>(vmx));
    vmx = qblock_max(fmaxf(vmx, dpp<kRowRor8>(vmx)));
    const int sv_new = prescale_exp(vmx, kSvTop);
    if (st.live) {
      const float f = __builtin_ldexpf(1.0f, sv_new - st.sv);
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
          st.acc[g][t][0] *= f;
          st.acc[g][t][1] *= f;
        }
    }
    st.sv = sv_new;
    st.vscale = __builtin_ldexpf(1.0f, sv_new);
    st.vhi = __builtin_ldexpf(1.0f, kSvTop - sv_new);
    st.vlo = __builtin_ldexpf(1.0f, kSvLow - sv_new);
  }
  {
    float2 k2 = br.ks, v2 = br.vs;
    k2.x *= kf;
    k2.y *= kf;
    v2.x *= st.vscale;
    v2.y *= st.vscale;
    *reinterpret_cast<float2*>(&sm.sks[wave][2 * lane]) = k2;
    *reinterpret_cast<float2*>(&sm.svs[wave][2 * lane]) = v2;
  }
  load_scales32(br, h, next, lo);  // next block's scales into the same registers
  const float us0 = us_row[0] * kun, us1 = us_row[1] * kun;

  // ---- S^T = codes^T * q~^T, 4 k-steps of 32 channels, two row tiles ------
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4 se[2] = {zero4, zero4}, so[2] = {zero4, zero4};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int c0 = ks * 32 + q * 8;
    const f32x4 sa = *reinterpret_cast<const f32x4*>(&sm.sks[wave][c0]);
    const f32x4 sb = *reinterpret_cast<const f32x4*>(&sm.sks[wave][c0 + 4]);
    float sk[8];  // k-slot order
    sk[0] = sa[0]; sk[1] = sa[2]; sk[2] = sa[1]; sk[3] = sa[3];
    sk[4] = sb[0]; sk[5] = sb[2]; sk[6] = sb[1]; sk[7] = sb[3];
    half2_t sk16[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sk16[i] = pk16(sk[2 * i], sk[2 * i + 1]);
    half8_t bh[2], bl[2];
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      half2_t q16[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) q16[i] = pk16(qk[t][ks][2 * i], qk[t][ks][2 * i + 1]);
      product_hilo(qk[t][ks], sk, q16, sk16, bh[t], bl[t]);
    }
    half8_t alo, ahi;  // tokens 2n and 2n + 1
    CodeOps<kBits>::to_half(br.k[ks], cc, alo, ahi);
    br.k[ks] = CodeOps<kBits>::load(h.kc, lo.k_off + ks * kKStep<kBits>,
                                    next * kBB<kBits>);  // next block's k-step
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      se[t] = mfma(alo, bh[t], se[t]);
      se[t] = mfma(alo, bl[t], se[t]);
      so[t] = mfma(ahi, bh[t], so[t]);
      so[t] = mfma(ahi, bl[t], so[t]);
    }
  }

  // raw[t][j]: row 16t + n, token 8q + j, in units of 2^Sq(row) (x kf)
  float raw[2][8];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      raw[t][2 * i] = se[t][i];
      raw[t][2 * i + 1] = so[t][i];
    }
    if (kMasked) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (tok0 + 8 * q + j >= t_end || (kCausal && tok0 + 8 * q + j > lim[t]))
          raw[t][j] = -INFINITY;
    }
  }
  const float us[2] = {us0, us1};
  float lmx[2];
#pragma unroll
  for (int t = 0; t < kTiles; ++t)
    lmx[t] = fmaxf(fmaxf(fmaxf(raw[t][0], raw[t][1]), fmaxf(raw[t][2], raw[t][3])),
                   fmaxf(fmaxf(raw[t][4], raw[t][5]), fmaxf(raw[t][6], raw[t][7]))) * us[t];

  // Move the reference of rows that overshoot it by more than kLazy (a
  // wave-uniform decision).
  if (!st.live || __builtin_amdgcn_ballot_w64(lmx[0] > st.m[0] + kLazy ||
                                              (kTiles > 1 && lmx[1] > st.m[1] + kLazy)) != 0) {
    float alpha[2];
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      const float mx = qblock_max(lmx[t]);  // row max over the block (finite unless kCausal)
      const float m_new = st.live ? (mx > st.m[t] + kLazy ? mx : st.m[t]) : mx;
      alpha[t] = st.live ? fast_exp2(st.m[t] - m_new) : 0.0f;
      if (kCausal && m_new == -INFINITY) alpha[t] = 0.0f;  // still no legal key: z = u = 0
      st.z[t] *= alpha[t];
      st.m[t] = m_new;
    }
    if (st.live) {
      // acc rows 16t + 4q + i take the factor of score row 16t + 4q + i,
      // owned by lanes n = 4q + i: exchange through this wave's LDS slot.
      if (q == 0) {
        sm.alp[wave][n] = alpha[0];
        if (kTiles > 1) sm.alp[wave][16 + n] = alpha[1];
      }
#pragma unroll
      for (int t = 0; t < kTiles; ++t) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(&sm.alp[wave][16 * t + 4 * q]);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          st.acc[g][t][0] *= a;
          st.acc[g][t][1] *= a;
        }
      }
    }
    st.live = true;
  }

  // p = 2^(s - m) <= 2^kLazy; z += sum p.  pk holds p in k-slot order.
  float pk[2][8];
  half2_t p16[2][4];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) {
    const float shift = kCausal && st.m[t] == -INFINITY ? 0.0f : -st.m[t];
    float pt[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) pt[j] = fast_exp2(fmaf(raw[t][j], us[t], shift));
    st.z[t] += ((pt[0] + pt[1]) + (pt[2] + pt[3])) + ((pt[4] + pt[5]) + (pt[6] + pt[7]));
#pragma unroll
    for (int j = 0; j < 8; ++j) pk[t][j] = pt[kSlotByte[j]];
#pragma unroll
    for (int i = 0; i < 4; ++i) p16[t][i] = pk16(pk[t][2 * i], pk[t][2 * i + 1]);
  }

  // ---- u += p~ x V codes, p~ = p * sV * 2^sv, one value group at a time ---
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const f32x4 va = *reinterpret_cast<const f32x4*>(&sm.svs[wave][g * 32 + q * 8]);
    const f32x4 vb = *reinterpret_cast<const f32x4*>(&sm.svs[wave][g * 32 + q * 8 + 4]);
    float sv[8];  // k-slot order
    sv[0] = va[0]; sv[1] = va[2]; sv[2] = va[1]; sv[3] = va[3];
    sv[4] = vb[0]; sv[5] = vb[2]; sv[6] = vb[1]; sv[7] = vb[3];
    half2_t sv16[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv16[i] = pk16(sv[2 * i], sv[2 * i + 1]);
    half8_t ah[2], al[2];
#pragma unroll
    for (int t = 0; t < kTiles; ++t) product_hilo(pk[t], sv, p16[t], sv16, ah[t], al[t]);
    half8_t be, bo;  // features 32g + 2n and 32g + 2n + 1
    CodeOps<kBits>::to_half(br.v[g], cc, be, bo);
    br.v[g] = CodeOps<kBits>::load(h.vc, lo.v_off + g * kVStep<kBits>,
                                   next * kBB<kBits>);  // next block's group
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      st.acc[g][t][0] = mfma(ah[t], be, st.acc[g][t][0]);
      st.acc[g][t][0] = mfma(al[t], be, st.acc[g][t][0]);
      st.acc[g][t][1] = mfma(ah[t], bo, st.acc[g][t][1]);
      st.acc[g][t][1] = mfma(al[t], bo, st.acc[g][t][1]);
    }
  }
}

// kTiles: 16-row tiles of query rows (1 for up to 16 rows per KV head, 2
// for up to 32).  kCausal: a causal chunk (row r is query r % R at position pos_end - R +
// r % R).  Only tokens past pos_end - R can be masked; they lie in at most
// two consecutive blocks (R <= 32), which belong to different waves and are
// each the last block of its wave.  So the masked block of a wave is the one
// it attends first, and its loop runs the unmasked path: every row reads
// every token there, which also gives a row still without a legal key its
// first one.
// kWindow: the last p.win_parts workgroups of each head attend recent-token
// window parts (a separate instantiation, so the plain kernel's block loop is
// compiled without that path).
template <int kBits, int kTiles, bool kCausal, bool kWindow>
__global__ __launch_bounds__(kT) __attribute__((amdgpu_waves_per_eu(2, 2))) void
attend_mfma_r32_kernel(AttendProblem p) {
  __shared__ Smem32 sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int q = lane >> 4;

  // Workgroup -> (KV head, split); all splits of a head on one XCD when the
  // head count allows (workgroups are dealt to the 8 XCDs round-robin).
  const int heads = p.B * p.Hkv;
  const int L = blockIdx.x;
  int head, split;
  if (heads % 8 == 0) {
    const int slot = L >> 3;
    head = (L & 7) + 8 * (slot / p.splits);
    split = slot % p.splits;
  } else {
    head = L / p.splits;
    split = L % p.splits;
  }
  const long long bh = head;
  const int rows = p.rows;
  const int packed_splits = p.splits - p.win_parts;
  if (kWindow && split >= packed_splits) {  // a window part (the whole workgroup)
    const int r = tid >> 3, f0 = (tid & 7) * 4;
    float U[16], M, Z;
    window_part<kR, kT, 16, 4, 32>(p, sm.u.win, bh, split - packed_splits, r, f0, U, M, Z);
    split_combine<16, 4, 32>(p, split, bh, r, f0, U, M, Z, &sm.last);
    return;
  }
  // Per-head strides follow the layout's capacity; only blocks below N are read.
  const int nblocks = (p.cap + kBlockTokens - 1) / kBlockTokens;
  Head32 h;
  h.kc = head_rsrc(p.k_codes + bh * nblocks * kBB<kBits>,
                   static_cast<long long>(nblocks) * kBB<kBits>);
  h.ksc = head_rsrc(p.k_scales + bh * nblocks * kBS, static_cast<long long>(nblocks) * kBS * 4);
  h.vc = head_rsrc(p.v_codes + bh * nblocks * kBB<kBits>,
                   static_cast<long long>(nblocks) * kBB<kBits>);
  h.vsc = head_rsrc(p.v_scales + bh * nblocks * kBS, static_cast<long long>(nblocks) * kBS * 4);

  const int t_begin = split * p.tokens_per_split;
  const int t_end = min(p.N, t_begin + p.tokens_per_split);
  const int b_begin = t_begin / kBlockTokens;
  const int b_end = t_end > t_begin ? (t_end + kBlockTokens - 1) / kBlockTokens : b_begin;
  const int b_first = b_begin + wave;
  const int b_last = b_first + (b_end - 1 - b_first) / kW * kW;  // valid if b_first < b_end
  // Code bytes of lane (n, q): K channels 32 ks + 8q .. +7 of tokens 2n, 2n + 1;
  // V tokens 8q .. 8q+7 of features 32 g + 2n, +1 (2 * kBits bytes each).
  const Lanes32 lo = {static_cast<unsigned>(lane * 2 * kBits),
                      static_cast<unsigned>(q * 128 * kBits + n * 2 * kBits),
                      static_cast<unsigned>(lane * 8)};

  // The block holding token N-1 is masked when N is not a multiple of 32;
  // the wave that owns it attends it first.  Its loads go out before the
  // query rows are staged.
  const bool active = b_first < b_end;
  const bool partial = ((p.N % kBlockTokens) != 0 && b_last == (p.N - 1) / kBlockTokens) ||
                       (kCausal && (b_last + 1) * kBlockTokens - 1 > p.pos_end - p.R);
  const int first = partial ? b_last : b_first;
  const int loop_begin = partial ? b_first : b_first + kW;
  const int loop_end = partial ? b_last - kW : b_last;  // inclusive
  Regs32<kBits> br;
  if (active) load_block32(br, h, first, lo);

  // q * qscale into LDS, each row prescaled by 2^Sq so its largest element
  // lies in [2^9, 2^10): thread -> (row tid >> 3, channels 16 (tid & 7) ..
  // +15).  Rows past `rows` are zero.
  {
    const int r = tid >> 3, c0 = (tid & 7) * 16;
    float v[16];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = 0.0f;
    if (r < rows) {
      const float* qrow = p.q + (bh * rows + r) * kD + c0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(qrow + 4 * i);
#pragma unroll
        for (int j = 0; j < 4; ++j) v[4 * i + j] = a[j] * p.qscale;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    amax = fmaxf(amax, __shfl_xor(amax, 4));
    const int sq = prescale_exp(amax, kQTop);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 a;
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = __builtin_ldexpf(v[4 * i + j], sq);
      *reinterpret_cast<f32x4*>(&sm.u.qs[r][c0 + 4 * i]) = a;
    }
    if ((tid & 7) == 0) sm.qus[r] = __builtin_ldexpf(1.0f, -sq);
  }
  __syncthreads();
  const float us_row[2] = {sm.qus[n], kTiles > 1 ? sm.qus[16 + n] : 1.0f};
  // This lane's q values for the whole kernel (rows 16t + n, channels
  // 32 ks + 8q + (0..7), k-slot order), kept in registers.
  float qk[2][4][8];
#pragma unroll
  for (int t = 0; t < kTiles; ++t)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const float* qrow = &sm.u.qs[16 * t + n][ks * 32 + q * 8];
      const f32x4 qa = *reinterpret_cast<const f32x4*>(qrow);
      const f32x4 qb = *reinterpret_cast<const f32x4*>(qrow + 4);
#pragma unroll
      for (int j = 0; j < 8; ++j) qk[t][ks][j] = j < 4 ? qa[kSlotByte[j]] : qb[kSlotByte[j] - 4];
    }

  const typename CodeOps<kBits>::consts cc = CodeOps<kBits>::make();
  State32 st;
  st.m[0] = st.m[1] = -INFINITY;
  st.z[0] = st.z[1] = 0.0f;
  st.sv = 0;
  st.vscale = 1.0f;
  st.vhi = st.vlo = 0.0f;
  st.live = false;
  {
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int t = 0; t < kTiles; ++t) st.acc[g][t][0] = st.acc[g][t][1] = zero4;
  }

  // Causal limit of this lane's score rows 16t + n.
  const int lim[2] = {p.pos_end - p.R + n % p.R, p.pos_end - p.R + (16 + n) % p.R};
  if (active) {
    attend_block32<kBits, kTiles, true, kCausal>(sm, br, first * kBlockTokens, t_end, cc, st, h,
                                  loop_begin <= loop_end ? loop_begin : first, lo, us_row, qk,
                                  lim);
    for (int b = loop_begin; b <= loop_end; b += kW)
      attend_block32<kBits, kTiles, false, false>(sm, br, b * kBlockTokens, t_end, cc, st, h,
                                   min(b + kW, loop_end), lo, us_row, qk, lim);
  }
  st.z[0] = qblock_sum(st.z[0]);
  if (kTiles > 1) st.z[1] = qblock_sum(st.z[1]);

  // ---- merge the waves: two at a time through LDS -------------------------
  // thread -> (row r = tid >> 3, features f0 + 32 i + (0..3), f0 = 4 (tid & 7))
  const int r = tid >> 3;
  const int f0 = (tid & 7) * 4;
  const float fu = __builtin_ldexpf(1.0f, -st.sv);
  __syncthreads();  // every wave is done with q (aliased by wu)
  if (q == 0) {
    sm.wm[wave][n] = st.m[0];
    sm.wm[wave][16 + n] = kTiles > 1 ? st.m[1] : -INFINITY;  // rows 16..31: none with one tile
    sm.wz[wave][n] = st.z[0];
    sm.wz[wave][16 + n] = kTiles > 1 ? st.z[1] : 0.0f;
  }
  float M = -INFINITY, Z = 0.0f;
  float U[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) U[i] = 0.0f;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if ((wave >> 1) == half) {  // waves 2 half, 2 half + 1 park their u
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int t = 0; t < kTiles; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float2 u2;
            u2.x = st.acc[g][t][0][i] * fu;
            u2.y = st.acc[g][t][1][i] * fu;
            *reinterpret_cast<float2*>(
                &sm.u.wu[wave & 1][16 * t + 4 * q + i][32 * g + 2 * n]) = u2;
          }
    }
    __syncthreads();
    if (half == 0) {
#pragma unroll
      for (int w = 0; w < kW; ++w) M = fmaxf(M, sm.wm[w][r]);
    }
    if (M != -INFINITY) {
#pragma unroll
      for (int w2 = 0; w2 < 2; ++w2) {
        const float mw = sm.wm[2 * half + w2][r];
        if (mw == -INFINITY) continue;
        const float e = fast_exp2(mw - M);
        Z = fmaf(e, sm.wz[2 * half + w2][r], Z);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(&sm.u.wu[w2][r][f0 + 32 * i]);
#pragma unroll
          for (int j = 0; j < 4; ++j) U[4 * i + j] = fmaf(e, a[j], U[4 * i + j]);
        }
      }
    }
    if (half == 0) __syncthreads();  // the first pair is read before the second overwrites it
  }
  const long long row0 = bh * rows;
  if (p.splits == 1) {
    if (r < rows) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = Z > 0.0f ? U[4 * i + j] / Z : 0.0f;  // Z = 0: no key
        *reinterpret_cast<f32x4*>(&p.out[(row0 + r) * kD + f0 + 32 * i]) = o;
      }
    }
    return;
  }

  split_combine<16, 4, 32>(p, split, bh, r, f0, U, M, Z, &sm.last);
}

}  // namespace

template <int kBits, int kTiles>
void launch_r32(const AttendProblem& p, unsigned grid, hipStream_t stream) {
  const bool win = p.win_parts > 0;
  if (p.causal) {
    if (win)
      hipLaunchKernelGGL((attend_mfma_r32_kernel<kBits, kTiles, true, true>), dim3(grid),
                         dim3(kT), 0, stream, p);
    else
      hipLaunchKernelGGL((attend_mfma_r32_kernel<kBits, kTiles, true, false>), dim3(grid),
                         dim3(kT), 0, stream, p);
  } else {
    if (win)
      hipLaunchKernelGGL((attend_mfma_r32_kernel<kBits, kTiles, false, true>), dim3(grid),
                         dim3(kT), 0, stream, p);
    else
      hipLaunchKernelGGL((attend_mfma_r32_kernel<kBits, kTiles, false, false>), dim3(grid),
                         dim3(kT), 0, stream, p);
  }
}

hipError_t launch_attend_mfma32(const AttendProblem& p, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>(p.splits) * p.B * p.Hkv;
  // One 16-row tile when the KV head has at most 16 query rows.
  if (p.bits == 8) {
    if (p.rows <= 16)
      launch_r32<8, 1>(p, grid, stream);
    else
      launch_r32<8, 2>(p, grid, stream);
  } else {
    if (p.rows <= 16)
      launch_r32<4, 1>(p, grid, stream);
    else
      launch_r32<4, 2>(p, grid, stream);
  }
  return hipGetLastError();
}

}  // namespace kvq
