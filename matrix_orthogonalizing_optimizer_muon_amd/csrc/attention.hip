// Causal softmax attention forward whose online-softmax running maximum also
// yields QK-Clip's per-head maximum logit ("MuonClip", section 05: the
// per-head signal is read off the forward's logits; "Muon and MuonClip:
// orthogonalised updates for LLM training", section 2, "The exploding-logit
// problem": the logits q.k/sqrt(d) that feed the softmax).  The maximum the
// softmax needs for stability is the statistic, so exporting it costs one
// wave reduction per 32 queries.
//
// Layout: Q, K, V, O bf16 [B][T][H][128]; lse fp32 [B][H][T].
// Block: 128 queries of one (batch row, head), 4 waves x 32 queries; keys in
// blocks of 64 staged through double-buffered LDS (K row-major, V transposed
// so the key index is contiguous for the P.V contraction).
// Per wave and key block, with v_mfma_f32_32x32x16_bf16:
//   S^T = K Q^T   (keys x queries: each lane owns one query column, so the
//                  row statistics are per-lane values plus one exchange with
//                  the lane 32 away)
//   O^T += V^T P^T (d x queries: the softmax rescale is a per-lane scalar)
// P takes the keys in the order its accumulator registers hold them; V^T is
// read in the same order, which leaves the contraction unchanged.
// The probabilities are exp2(s c2 - r) against a reference r that moves only
// when a query's running maximum passes it by more than 8 (in log2 units):
// the ratio O = sum p v / sum p does not depend on r, p stays below 2^8, and
// the rescale of O and of the running sum is skipped for most key blocks.
// The exact running maximum is still kept for the statistic.
#include <cmath>

#include "common.hpp"

namespace muon {

namespace {

typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

constexpr int kD = 128;        // head dimension
constexpr int kQB = 128;       // queries per block
constexpr int kKB = 64;        // keys per iteration
constexpr int kKP = kD + 8;    // K tile row pitch (bf16), 272 bytes
constexpr int kVP = kKB + 4;   // V^T tile row pitch (bf16), 136 bytes: conflict-free 8-byte reads

__device__ __forceinline__ float wave_max64(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

template <bool CAUSAL>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(AttnArgs A) {
  __shared__ __attribute__((aligned(16))) bf16_t sK[2][kKB * kKP];
  __shared__ __attribute__((aligned(16))) bf16_t sVt[2][kD * kVP];

  // Each XCD (block b runs on XCD b % 8) owns a contiguous range of heads and
  // walks it in groups of 4 heads, the group's query blocks heaviest first
  // (longest causal rows first across the group): the heads of a group share
  // that XCD's L2 for their K and V, and the short blocks fill the end of each
  // group.  Head counts that do not split that way fall back to one head's
  // query blocks at a time.
  int bh, qb;
  if (!xcd_group_order(blockIdx.x, A.B * A.H, A.nqb, 4, &bh, &qb)) {
    const int lin = xcd_remap(blockIdx.x, gridDim.x);
    bh = lin / A.nqb;
    qb = A.nqb - 1 - (lin - bh * A.nqb);
  }
  const int b = bh / A.H, head = bh - b * A.H;
  const int T = A.T;
  const int64_t tok = static_cast<int64_t>(A.H) * kD;                 // token stride
  const int64_t base = (static_cast<int64_t>(b) * T * A.H + head) * kD;  // (b, t=0, head, 0)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hf = lane >> 5;     // lane half: which 8 of each 16 contraction slots
  const int col = lane & 31;
  const int q0w = qb * kQB + 32 * wave;
  const int q = q0w + col;

  // this lane's query as the B operand of S^T = K Q^T, all 8 slices of d
  bf16x8_t qf[kD / 16];
  static_for<kD / 16>([&](auto kc) {
    if (q < T) qf[kc] = *reinterpret_cast<const bf16x8_t*>(A.Q + base + q * tok + 16 * kc + 8 * hf);
    else qf[kc] = bf16x8_t{};
  });

  const int kend = CAUSAL ? min(T, qb * kQB + kQB) : T;
  const int nkb = (kend + kKB - 1) / kKB;
  int wkb_end = 0;              // key blocks this wave needs
  if (q0w < T) wkb_end = CAUSAL ? (min(T - 1, q0w + 31) / kKB + 1) : nkb;

  // ---- staging: K 64 x 128 as 4 x 16 bytes per thread; V 2 passes x 2 keys x 16 bytes
  u32x4_t kr[4], vr[2][2];
  const int krow = tid >> 4, kcc = tid & 15;
  const int vkp = tid & 31, vdc = tid >> 5;
  auto gload = [&](int kb) {
    const int k0 = kb * kKB;
    static_for<4>([&](auto i) {
      const int key = k0 + krow + 16 * i;
      kr[i] = key < T ? *reinterpret_cast<const u32x4_t*>(A.K + base + key * tok + 8 * kcc) : u32x4_t{};
    });
    static_for<2>([&](auto p) {
      const int d0 = 8 * (vdc + 8 * p);
      static_for<2>([&](auto j) {
        const int key = k0 + 2 * vkp + j;
        vr[p][j] = key < T ? *reinterpret_cast<const u32x4_t*>(A.V + base + key * tok + d0) : u32x4_t{};
      });
    });
  };
  auto sstore = [&](int buf) {
    static_for<4>([&](auto i) {
      *reinterpret_cast<u32x4_t*>(&sK[buf][(krow + 16 * i) * kKP + 8 * kcc]) = kr[i];
    });
    static_for<2>([&](auto p) {
      const int d0 = 8 * (vdc + 8 * p);
      static_for<4>([&](auto wi) {
        constexpr int w = decltype(wi)::value;
        // d0 + 2w and d0 + 2w + 1 from the two keys 2 vkp, 2 vkp + 1
        const uint32_t a = vr[p][0][w], c = vr[p][1][w];
        *reinterpret_cast<uint32_t*>(&sVt[buf][(d0 + 2 * w) * kVP + 2 * vkp]) = (a & 0xffffu) | (c << 16);
        *reinterpret_cast<uint32_t*>(&sVt[buf][(d0 + 2 * w + 1) * kVP + 2 * vkp]) = (a >> 16) | (c & 0xffff0000u);
      });
    });
  };
  // LDS-only barrier: the prefetch loads stay in flight across it
  auto barrier = [&]() { lds_barrier(); };

  f32x16_t o[kD / 32];
  static_for<kD / 32>([&](auto i) { o[i] = f32x16_t{}; });
  float m_run = -INFINITY, l_run = 0.0f;
  float mref = -INFINITY;   // exponent reference: m_run * c2 <= mref + 8
  int nanf = 0;
  const float c2 = A.c2;

  auto compute = [&](int buf, int kb) {
    const int k0 = kb * kKB;
    f32x16_t s[2] = {f32x16_t{}, f32x16_t{}};
    const bf16_t* kb0 = &sK[buf][col * kKP + 8 * hf];
    static_for<kD / 16>([&](auto kc) {
      const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(kb0 + 16 * kc);
      const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(kb0 + 32 * kKP + 16 * kc);
      s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[kc], s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[kc], s[1], 0, 0, 0);
    });
    // key of accumulator element e of block mb: k0 + 32 mb + 8 (e / 4) + 4 hf + e % 4
    const bool need_mask = (k0 + kKB > T) || (CAUSAL && k0 + kKB - 1 > q0w);
    float mloc = -INFINITY;
    if (need_mask) {
      static_for<32>([&](auto i) {
        constexpr int MB = decltype(i)::value / 16, E = decltype(i)::value % 16;
        const int key = k0 + 32 * MB + 8 * (E / 4) + 4 * hf + (E % 4);
        const bool ok = key < T && (!CAUSAL || key <= q);
        s[MB][E] = ok ? s[MB][E] : -INFINITY;
      });
    }
    // IEEE maximum propagates NaN (v_maximum3_f32: two logits per instruction)
    static_for<16>([&](auto i) {
      constexpr int MB = decltype(i)::value / 8, E = 2 * (decltype(i)::value % 8);
      mloc = __builtin_elementwise_maximum(mloc, __builtin_elementwise_maximum(s[MB][E], s[MB][E + 1]));
    });
    nanf |= (mloc != mloc);
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    m_run = fmaxf(m_run, mloc);
    // move the exponent reference (and rescale) only where the maximum has
    // passed it by more than 8; one wave-wide test per key block
    const float mn2 = m_run * c2;
    const bool up = mn2 > mref + 8.0f;
    if (__builtin_amdgcn_ballot_w64(up) != 0) {
      const float nref = up ? mn2 : mref;
      const float alpha = (mref == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mref - nref);
      mref = nref;
      l_run *= alpha;
      static_for<kD / 32>([&](auto i) { o[decltype(i)::value] = o[decltype(i)::value] * alpha; });
    }
    const float mc = (mref == -INFINITY) ? 0.0f : mref;
    bf16x8_t pb[4];
    static_for<32>([&](auto i) {
      constexpr int MB = decltype(i)::value / 16, E = decltype(i)::value % 16;
      const float p = __builtin_amdgcn_exp2f(fmaf(s[MB][E], c2, -mc));
      l_run += p;
      s[MB][E] = p;
    });
    static_for<4>([&](auto cc) {
      constexpr int C = decltype(cc)::value;
      f32x8_t pv;
      static_for<8>([&](auto j) {
        constexpr int J = decltype(j)::value;
        pv[J] = s[C / 2][8 * (C % 2) + J];
      });
      pb[C] = __builtin_convertvector(pv, bf16x8_t);   // v_cvt_pk_bf16_f32: nearest-even
    });
    // O^T += V^T P^T; slot j of lane half hf is key 16 c + 8 (j / 4) + 4 hf + j % 4
    static_for<4>([&](auto cc) {
      constexpr int C = decltype(cc)::value;
      static_for<kD / 32>([&](auto db) {
        const bf16_t* vrow = &sVt[buf][(32 * db + col) * kVP + 16 * C + 4 * hf];
        const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(vrow);
        const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(vrow + 8);
        const u32x4_t w = {lo[0], lo[1], hi[0], hi[1]};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w), pb[C], o[db], 0, 0, 0);
      });
    });
  };

  gload(0);
  sstore(0);
  if (nkb > 1) gload(1);
  barrier();
  for (int kb = 0; kb < nkb; ++kb) {
    const int cur = kb & 1;
    if (kb < wkb_end) compute(cur, kb);
    if (kb + 1 < nkb) {
      sstore(cur ^ 1);
      if (kb + 2 < nkb) gload(kb + 2);
    }
    barrier();
  }

  // ---- epilogue: normalise, store O and lse, export this wave's maximum logit
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  if (q < T) {
    bf16_t* orow = A.O + base + q * tok;
    static_for<kD / 32>([&](auto db) {
      static_for<4>([&](auto g) {
        constexpr int G = decltype(g)::value;
        const int d0 = 32 * db + 8 * G + 4 * hf;
        u32x2_t pk;
        constexpr int DB = decltype(db)::value;
        const f32x4_t ov = {o[DB][4 * G] * inv, o[DB][4 * G + 1] * inv, o[DB][4 * G + 2] * inv,
                            o[DB][4 * G + 3] * inv};
        pk = __builtin_bit_cast(u32x2_t, __builtin_convertvector(ov, bf16x4_t));
        *reinterpret_cast<u32x2_t*>(orow + d0) = pk;
      });
    });
    if (A.lse && hf == 0)
      A.lse[(static_cast<int64_t>(b) * A.H + head) * T + q] =
          (mref == -INFINITY ? 0.0f : mref * 0.69314718055994531f) + logf(l_tot);   // r ln 2 = (r / c2) scale
  }
  const float mw = wave_max64(q < T ? m_run : -INFINITY);
  const int anynan = __any(q < T && nanf);
  if (lane == 0)
    A.partial[((static_cast<int64_t>(b) * A.H + head) * A.nqb + qb) * 4 + wave] =
        anynan ? __uint_as_float(0x7fc00000u) : mw;
}

}  // namespace

hipError_t launch_attn_fwd(const AttnArgs& A, int causal, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(A.B) * A.H * A.nqb), block(256);
  if (causal) hipLaunchKernelGGL(attn_fwd_kernel<true>, grid, block, 0, s, A);
  else hipLaunchKernelGGL(attn_fwd_kernel<false>, grid, block, 0, s, A);
  return hipGetLastError();
}

}  // namespace muon
