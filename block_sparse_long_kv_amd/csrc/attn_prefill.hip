// Block-sparse causal prefill attention on bf16 MFMA (fp32 accumulate).
//
// Source: "SparDA: a fourth projection that lets sparse attention prefetch
// its own KV cache" -- "The fourth projection", Eq. 5 and Alg. 1 (attention
// of the chunk's queries over the K/V of each query block's selected blocks).
//
// Design (gfx950, v_mfma_f32_16x16x32_bf16):
//   * One workgroup per (query block of 64 tokens, KV head, group of up to 4
//     query heads): for HPW heads it runs 2*HPW wavefronts, each serving 32
//     query rows of one head, so those heads share every K/V block staged in
//     LDS.
//   * Scores are computed transposed, S^T = K Q^T (keys on the MFMA M side):
//     the accumulator layout then gives each lane one query column, so the
//     online-softmax statistics and the probabilities stay in the lane that
//     owns them, and P^T feeds O^T = V^T P^T as the B operand directly.
//   * Ping-pong between two wave groups.  Group A (rows 0..31 of every head)
//     and group B (rows 32..63) run the same schedule one slot apart: in a
//     slot a wave either issues MFMAs (S for block a and O += V^T P for block
//     a-1) or runs the softmax of block a.  Waves w and w+HPW share a SIMD, so
//     each SIMD always has one wave on the matrix cores while the other keeps
//     the VALU busy; one barrier closes each slot.
//   * K and V live in LDS rings (four stages each with four heads per
//     workgroup, else two) filled by gfx950's global-to-LDS copies
//     (global_load_lds_dwordx4): no registers hold the blocks in transit and
//     no LDS writes are issued, and with four stages a block's copy is issued
//     four slots before its first read.  With four heads per workgroup group
//     B issues every copy, in its softmax slots, so the MFMA slots carry no
//     copy work (774-780 vs 786-792 us per B4 x 128K chunk with each wave
//     copying its share, the MFMA group included); the smaller forms keep
//     every wave copying.  Rows are unpadded (a copy writes
//     1024 contiguous bytes) with 16-byte chunks XOR-swizzled per row, which
//     keeps the K fragment reads and the transposing V reads
//     (ds_read_b64_tr_b16, two per operand) free of extra bank conflicts.
//   * Online softmax with a lazy maximum: the running maximum only moves when
//     a row's block maximum exceeds it by more than 8 (base-2 units), so the
//     output is rarely rescaled; probabilities stay below 2^8, which fp32
//     accumulation and bf16 operands carry without loss of relative accuracy.
//     The test runs on each lane's own maximum, so the common case needs no
//     cross-lane traffic; row sums are kept per lane and reduced once at the
//     end.
//   * Workgroups are ordered so that consecutive query blocks of one KV head
//     run on the same XCD: neighbouring query blocks share most of their
//     local-window blocks, which then hit in that XCD's L2.
#include "bskv_device.hpp"
#include "bskv_launch.hpp"

namespace bskv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& r) { return __builtin_bit_cast(bf16x8_t, r); }

// Two workgroups per CU for one and two heads per workgroup (two LDS stages
// each), one for four (four stages, 128 KB); at head_dim 128 the one-head
// form needs ~390 registers per lane (its 8 copy pieces per wave and tile add
// address registers), so it runs one wave per SIMD and is declared so.
template <int D, int HPW>
__global__ __launch_bounds__(HPW * 128, (HPW == 1 && D == 128) ? 1 : 2) void attn_prefill_kernel(
    const bf16_bits* __restrict__ q, const bf16_bits* __restrict__ k, const bf16_bits* __restrict__ v, int64_t sb,
    int64_t sg, int64_t st, int64_t kv_len, const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt,
    int64_t q_start, int Tq, int Hkv, int G, int U, int n_qb, float qscale, bf16_bits* __restrict__ out) {
  constexpr int BLK = 64;
  constexpr int NT = HPW * 128;        // threads: 2*HPW waves
  constexpr int NW = NT / 64;
  constexpr int RB = D * 2;            // bytes per K/V row
  constexpr int RCH = D / 8;           // 16-byte chunks per row
  constexpr int TILE = BLK * RB;       // bytes of one K or V block
  // the waves that copy K/V tiles: group B's with four heads per workgroup
  // (the MFMA slots then carry no copy work), every wave otherwise (fewer
  // copy pieces per wave: the two-head form would spill registers)
  constexpr bool B_COPIES = HPW == 4;
  constexpr int NCW = B_COPIES ? NW / 2 : NW;
  constexpr int PPW = TILE / 1024 / NCW;  // 1024-byte copy pieces per copying wave per tile
  static_assert(PPW >= 1 && PPW * NCW * 1024 == TILE, "copy pieces");
  // ring stages: four (a copy is issued four slots before its block is
  // read) for four heads per workgroup, two otherwise (so that two
  // workgroups still share a CU)
  constexpr int NST = HPW == 4 ? 4 : 2;
  constexpr int KS = D / 32;           // k-steps of S^T
  constexpr int MD = D / 16;           // d tiles of O^T
  constexpr float TAU = 8.f;           // lazy-maximum threshold (base 2)
  // Unpadded rows with 16-byte chunks XOR-swizzled per row (the copies write
  // whole 1024-byte pieces, so rows cannot be padded): K chunk c of row r
  // sits at chunk c ^ (r % RCH), V chunk c at c ^ 2 (r % MD).  Both keep the
  // MFMA fragment reads below at the bank-conflict level of padded rows.
  __shared__ __attribute__((aligned(1024))) unsigned char Ks[NST][TILE];
  __shared__ __attribute__((aligned(1024))) unsigned char Vs[NST][TILE];

  const int n_tiles = gridDim.x;
  int lin = blockIdx.x;
  if ((n_tiles & 7) == 0) lin = (lin & 7) * (n_tiles >> 3) + (lin >> 3);
  const int n_hs = G / HPW;
  const int qi = lin % n_qb, rest = lin / n_qb;
  const int hs = rest % n_hs, bg = rest / n_hs;
  const int b = bg / Hkv, g = bg % Hkv;
  const int Hq = Hkv * G;
  // the wave index is made wave-uniform for the compiler, so that every
  // slot branch below is scalar and the block list is read with scalar loads
  const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wid / HPW;           // 0: group A, 1: group B (one slot later)
  const int h = g * G + hs * HPW + wid % HPW;
  const int row0 = grp * 32;
  const int l16 = lane & 15, lg = lane >> 4;
  const int qb = (int)(q_start / BLK) + qi;
  const int tq0 = qi * BLK;

  // no block lies inside K/V shorter than one block: every query row has
  // nothing to attend to and its output is zero
  if (kv_len < BLK) {
#pragma unroll
    for (int nq = 0; nq < 2; ++nq) {
      const int t = tq0 + row0 + 16 * nq + l16;
      if (t < Tq) {
        bf16_bits* op = out + (((int64_t)b * Hq + h) * Tq + t) * D + 4 * lg;
#pragma unroll
        for (int md = 0; md < MD; ++md) *reinterpret_cast<uint2*>(op + 16 * md) = make_uint2(0, 0);
      }
    }
    return;
  }

  // Q^T fragments (B operand of S^T): query rows row0 + 16*nq + l16
  bf16x8_t qf[2][KS];
#pragma unroll
  for (int nq = 0; nq < 2; ++nq) {
    const int t = tq0 + row0 + 16 * nq + l16;
    const bf16_bits* qp = q + (((int64_t)b * Hq + h) * Tq + t) * D + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 r = make_uint4(0, 0, 0, 0);
      if (t < Tq) r = ld16(qp + 32 * ks);
      qf[nq][ks] = as_bf16x8(r);
    }
  }

  f32x4_t o[MD][2];
#pragma unroll
  for (int md = 0; md < MD; ++md)
#pragma unroll
    for (int nq = 0; nq < 2; ++nq) o[md][nq] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t s[4][2];
  bf16x8_t pb[2][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nq = 0; nq < 2; ++nq) s[mt][nq] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int nq = 0; nq < 2; ++nq) pb[s2][nq] = as_bf16x8(make_uint4(0, 0, 0, 0));
  // running max (base-2, scaled) starts finite: a fully masked block then
  // gives p = 0 without special cases; the row sum is a per-lane partial
  float m_run[2] = {-1e30f, -1e30f}, l_part[2] = {0.f, 0.f};

  // The Q fragments have arrived before any copy is issued (vmcnt 0); the
  // compiler, which does not see the copies, then places no wait for them
  // inside the slot loop, where it would also wait for the copies in flight.
  __builtin_amdgcn_s_waitcnt(0x0F70);

  const int64_t prob = (int64_t)bg * n_qb + qi;
  const int c = min(cnt[prob], U);
  // the block list is read through the constant address space: uniform
  // indices then give scalar loads, which do not wait behind the copies in
  // flight (vector memory operations complete in order)
  const __attribute__((address_space(4))) int32_t* list =
      (const __attribute__((address_space(4))) int32_t*)(idx + prob * U);
  const bf16_bits* kb = k + b * sb + g * sg;
  const bf16_bits* vb = v + b * sb + g * sg;

  // a listed block is used only if it lies inside the K/V buffers; a block
  // outside them is masked whole and its copy reads block 0 instead (K/V
  // hold at least one block here), so the stage holds finite values
  auto valid = [&](int jj) { return jj >= 0 && ((int64_t)jj + 1) * BLK <= kv_len; };
  // this lane's share of a tile: piece (wid - HPW)*PPW + i (group B copying)
  // or wid*PPW + i (every wave) covers LDS chunks 64 piece + lane, i.e. row
  // r, stored chunk cs; the global chunk is the logical one, cs ^ swizzle(r)
  const uint32_t ks_base = lds_u32(&Ks[0][0]), vs_base = lds_u32(&Vs[0][0]);
  auto copy_tile = [&](const bf16_bits* base, uint32_t lds_stage, int jj, bool is_v) {
    const bf16_bits* p0 = base + (int64_t)(valid(jj) ? jj : 0) * BLK * st;
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
      const int piece = (B_COPIES ? wid - HPW : wid) * PPW + i;
      const int qc = piece * 64 + lane, r = qc / RCH, cs = qc % RCH;
      const int cl = cs ^ (is_v ? 2 * (r % MD) : r % RCH);
      lds_dma16(p0 + (int64_t)r * st + cl * 8, __builtin_amdgcn_readfirstlane(lds_stage + piece * 1024));
    }
  };
  // copies issued at the start of even slot 2m: V(m-2+NST), then
  // K(m-1+NST), into the stages their blocks' predecessors left in slot 2m-1
  auto issue = [&](int m) {
    const int jv = m - 2 + NST, jk = m - 1 + NST;
    if (jv >= 0 && jv < c) copy_tile(vb, vs_base + (jv % NST) * TILE, list[jv], true);
    if (jk >= 0 && jk < c) copy_tile(kb, ks_base + (jk % NST) * TILE, list[jk], false);
  };
  // before the barrier that opens slot 2m: K(m) and V(m-1) have landed.  They
  // were issued in slot 2(m-NST+1); every later slot issued 2 PPW copies
  // while the blocks exist, else nothing is left in flight that matters.
  auto wait_copies = [&](int m) {
    if (m + NST - 2 < c) wait_vm<2 * (NST - 2) * PPW>();
    else wait_vm<0>();
  };

  // per-lane LDS byte offsets of the fragment reads
  int kofs[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) kofs[ks] = l16 * RB + 16 * ((4 * ks + lg) ^ (l16 % RCH));
  const int tr_row = 4 * lg + (l16 >> 2), tr_col = 4 * (l16 & 3);
  const int vrow = tr_row * RB + 16 * (tr_col >> 3) + 2 * (tr_col & 7), vsw = tr_row % MD;

  // MFMA slot: S^T = K(a) Q^T (a < c) and O^T += V(a-1)^T P(a-1)^T (a >= 1)
  auto mfma_slot = [&](int a) {
    if (a < c) {
      const unsigned char* kst = &Ks[a % NST][0];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nq = 0; nq < 2; ++nq) s[mt][nq] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const bf16x8_t a_op = as_bf16x8(*reinterpret_cast<const uint4*>(kst + kofs[ks] + mt * 16 * RB));
#pragma unroll
          for (int nq = 0; nq < 2; ++nq)
            s[mt][nq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_op, qf[nq][ks], s[mt][nq], 0, 0, 0);
        }
      }
    }
    if (a >= 1) {
      // The V^T operand (lane: d = 16*md + l16, keys 32*s2 + 4*lg + {0..3} and
      // 32*s2 + 16 + 4*lg + {0..3}) comes from row-major V with transposing LDS
      // reads: within each 16-lane group, lane 4r+c reads key row r, columns
      // 4c..4c+3, and ds_read_b64_tr_b16 hands lane i element i%4 of lane
      // 4r+i/4 for r = 0..3.  Rows 32*s2 + tr_row and 16 below it share the
      // row swizzle, so only the d tile's chunk pair moves: md ^ (row % MD).
      const unsigned char* vst = &Vs[(a - 1) % NST][0];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
        for (int md = 0; md < MD; ++md) {
          const unsigned char* v0 = vst + 32 * s2 * RB + vrow + 32 * (md ^ vsw);
          const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)v0);
          const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(v0 + 16 * RB));
          const bf16x8_t a_op =
              __builtin_bit_cast(bf16x8_t, s16x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
#pragma unroll
          for (int nq = 0; nq < 2; ++nq)
            o[md][nq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_op, pb[s2][nq], o[md][nq], 0, 0, 0);
        }
      }
    }
  };

  // softmax slot of block a: S -> P (bf16 operand), running max and sum
  auto softmax_slot = [&](int a) {
    const int j = list[a];
    // causal mask: the diagonal block per token (uniform over the
    // workgroup); a listed block after the query block, or outside the
    // buffers, is masked whole
    if (j >= qb || !valid(j)) {
      const bool ok = valid(j) && j == qb;
#pragma unroll
      for (int nq = 0; nq < 2; ++nq) {
        const int rq = row0 + 16 * nq + l16;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (!ok || 16 * mt + 4 * lg + i > rq) s[mt][nq][i] = -INFINITY;
      }
    }
#pragma unroll
    for (int nq = 0; nq < 2; ++nq) {
      float mx = s[0][nq][0];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[mt][nq][i]);
      // The lane-local maximum decides whether the running maximum must move:
      // usually no lane exceeds it by more than TAU and nothing crosses lanes.
      // Otherwise the four lanes of each query column agree on the column
      // maximum and the columns that moved rescale their output and sum.
      if (__any(mx * qscale > m_run[nq] + TAU)) {
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float ms = mx * qscale;
        const bool up = ms > m_run[nq] + TAU;
        const float alpha = up ? __builtin_amdgcn_exp2f(m_run[nq] - ms) : 1.f;
        m_run[nq] = up ? ms : m_run[nq];
        l_part[nq] *= alpha;
#pragma unroll
        for (int md = 0; md < MD; ++md) o[md][nq] *= alpha;
      }
      const float mn = m_run[nq];
      float sum = 0.f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][nq][i], qscale, -mn));
          s[mt][nq][i] = p;
          sum += p;
        }
      l_part[nq] += sum;
      // P^T operand for key step s2: slots 0..3 <- tile 2*s2, slots 4..7 <- tile 2*s2+1
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        bf16x8_t p8;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p8[e] = (__bf16)s[2 * s2][nq][e];
          p8[4 + e] = (__bf16)s[2 * s2 + 1][nq][e];
        }
        pb[s2][nq] = p8;
      }
    }
  };

  // Slots: group A runs M(0) S(0) M(1) S(1) ... S(c-1) M(c) in slots 0..2c,
  // group B the same sequence in slots 1..2c+1, where M(a) is the MFMA slot
  // of block a and S(a) its softmax slot; one barrier closes each slot.  K(u)
  // is read in slots 2u and 2u+1, V(u) in slots 2u+2 and 2u+3.  The copying
  // waves (group B with four heads, where it runs S(m-1) or, m = 0, idles;
  // else every wave) issue their share of each tile at the start of even
  // slot 2m: V(m-2+NST) and K(m-1+NST) go into the stages of V(m-2) and
  // K(m-1), last read in slot 2m-1; before the barrier closing slot 2m-1
  // each copying wave waits for its copies of K(m) and V(m-1), so after
  // that barrier every wave may read them.  The prologue issues the copies
  // of the slots before 0 (K(0..NST-2), V(0..NST-3)) and waits for K(0).
  if (!B_COPIES || grp == 1) {
#pragma unroll
    for (int m = 1 - NST; m < 0; ++m) issue(m);
    wait_copies(0);
  }
  __syncthreads();
  if (grp == 1) {                      // slot 0: group B idle
    issue(0);
    __syncthreads();
  }
  for (int a = 0;; ++a) {
    if (!B_COPIES && grp == 0) issue(a);   // A: slot 2a
    __builtin_amdgcn_s_setprio(1);
    mfma_slot(a);
    __builtin_amdgcn_s_setprio(0);
    if (grp == 1) wait_copies(a + 1);  // B: slot 2a+1 closes
    __syncthreads();
    if (a == c) break;
    if (grp == 1) issue(a + 1);        // B: slot 2a+2
    softmax_slot(a);
    if (!B_COPIES && grp == 0) wait_copies(a + 1);   // A: slot 2a+1 closes
    __syncthreads();
  }
  if (grp == 0) __syncthreads();       // slot 2c+1: group A idle

  // epilogue: O[query][d] = O^T[d][query] / l
#pragma unroll
  for (int nq = 0; nq < 2; ++nq) {
    float l = l_part[nq];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int t = tq0 + row0 + 16 * nq + l16;
    if (t < Tq) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      bf16_bits* op = out + (((int64_t)b * Hq + h) * Tq + t) * D + 4 * lg;
#pragma unroll
      for (int md = 0; md < MD; ++md) {
        const uint32_t w0 = (uint32_t)f32_to_bf16(o[md][nq][0] * inv) | ((uint32_t)f32_to_bf16(o[md][nq][1] * inv) << 16);
        const uint32_t w1 = (uint32_t)f32_to_bf16(o[md][nq][2] * inv) | ((uint32_t)f32_to_bf16(o[md][nq][3] * inv) << 16);
        *reinterpret_cast<uint2*>(op + 16 * md) = make_uint2(w0, w1);
      }
    }
  }
}

template <int D, int HPW>
static void launch_prefill_t(const AttnPrefillArgs& a) {
  const int G = a.Hq / a.Hkv;
  const int n_qb = (a.Tq + 63) / 64;
  const int n_tiles = n_qb * a.B * a.Hkv * (G / HPW);
  const float qscale = a.scale * 1.4426950408889634f;
  hipLaunchKernelGGL((attn_prefill_kernel<D, HPW>), dim3(n_tiles), dim3(HPW * 128), 0, a.stream, (const bf16_bits*)a.q,
                     (const bf16_bits*)a.k, (const bf16_bits*)a.v, a.sb, a.sg, a.st, a.kv_len, a.idx, a.cnt, a.q_start, a.Tq,
                     a.Hkv, G, a.U, n_qb, qscale, (bf16_bits*)a.out);
}

template <int D>
static void launch_prefill_d(const AttnPrefillArgs& a, int G) {
  switch (G) {
    case 1: launch_prefill_t<D, 1>(a); break;
    case 2: launch_prefill_t<D, 2>(a); break;
    default: launch_prefill_t<D, 4>(a); break;   // G = 4 or 8: four query heads per workgroup
  }
}

hipError_t launch_attn_prefill(const AttnPrefillArgs& a) {
  const int G = a.Hq / a.Hkv;
  if (a.D == 64) launch_prefill_d<64>(a, G);
  else launch_prefill_d<128>(a, G);
  return hipGetLastError();
}

}  // namespace bskv
