// gdr_fwd.hip -- forward kernels of the chunked gated delta rule on gfx950.
//
// Chunk form (derived from the recurrence S_t = e^{g_t}(I - b_t k_t k_t^T)S_{t-1}
// + b_t k_t v_t^T, o_t = s S_t^T q_t; the pages name the WY intermediates
// W, U and the per-chunk state S that the forward writes and re-reads:
// FlashQLA curated summary, section "GDN Chunked Prefill的效率問題").  For a
// chunk of n <= 64 tokens entering with state h:
//   gamma = cumsum(g),  Gamma = e^gamma,  D_ij = e^{gamma_i - gamma_j}
//   L = strict_lower(diag(b) (D * K K^T)),  A = (I + L)^{-1}
//   W = A diag(b Gamma) K,   U = A diag(b) V,   Vnew = U - W h
//   O = s (diag(Gamma) Q h + lower(D * Q K^T) Vnew)
//   h' = Gamma_n h + (diag(e^{gamma_n - gamma}) K)^T Vnew
//
// Kernels, in launch order:
//   k_plan    token/chunk/segment offset tables (one workgroup)
//   k_intra_w per (chunk, value head), one item per wave (bf16): gate
//             cumsum, K K^T, blocked fp32 triangular inverse, A diag(beta)
//             rows                                           [fully parallel]
//   k_intra   the same per workgroup for fp32, storing W and U instead
//   k_fused   per (sequence, value head, CP segment): the serial chunk
//             recurrence with h in fp32 registers, fused with O  [serial part]
//   (k_state  the same recurrence storing every chunk's entry state, for the
//             backward's recompute)
// The split of the serial state pass into context-parallel segments rebuilt
// by a gate-decay warmup follows the pages' automatic single-card CP (FlashQLA
// curated summary, section "平衡解決方案：雙核心融合與自動CP"; Tongyi page,
// section "FlashQLAの主な利点").
#include <math.h>
#include <algorithm>
#include <type_traits>

#include "gdr_device.h"
#include "gdr_kernels.h"

namespace gdr {

// ---------------------------------------------------------------- k_plan --
// cu[n] (copied or n*T), chunk_off[n] = sum_{m<n} ceil(len_m / 64),
// seg_off[n] = sum_{m<n} max(1, ceil(chunks_m / seg_chunks)).
__global__ __launch_bounds__(1024) void k_plan(PlanParams p) {
  __shared__ int32_t sc[2][1024], ss[2][1024];
  const int tid = threadIdx.x, N = p.N;
  const int per = (N + 1023) / 1024;
  const int b = min(tid * per, N), e = min(b + per, N);
  auto cu_at = [&](int n) -> int32_t { return p.cu_in ? p.cu_in[n] : n * p.T; };
  int c_sum = 0, s_sum = 0;
  for (int n = b; n < e; ++n) {
    const int len = max(cu_at(n + 1) - cu_at(n), 0);
    const int ch = (len + CH - 1) / CH;
    c_sum += ch;
    s_sum += max(1, (ch + p.seg_chunks - 1) / p.seg_chunks);
  }
  int buf = 0;
  sc[0][tid] = c_sum;
  ss[0][tid] = s_sum;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {  // inclusive Hillis-Steele scan
    const int a = sc[buf][tid] + (tid >= d ? sc[buf][tid - d] : 0);
    const int s2 = ss[buf][tid] + (tid >= d ? ss[buf][tid - d] : 0);
    buf ^= 1;
    sc[buf][tid] = a;
    ss[buf][tid] = s2;
    __syncthreads();
  }
  int c_run = sc[buf][tid] - c_sum, s_run = ss[buf][tid] - s_sum;  // exclusive
  for (int n = b; n < e; ++n) {
    const int len = max(cu_at(n + 1) - cu_at(n), 0);
    const int ch = (len + CH - 1) / CH;
    p.cu[n] = cu_at(n);
    p.chunk_off[n] = c_run;
    p.seg_off[n] = s_run;
    c_run += ch;
    s_run += max(1, (ch + p.seg_chunks - 1) / p.seg_chunks);
  }
  if (tid == 1023) {
    p.cu[N] = cu_at(N);
    p.chunk_off[N] = sc[buf][1023];
    p.seg_off[N] = ss[buf][1023];
  }
  if (p.seg_order) {
    // Segments by decreasing work (its chunks plus the warmup chunks before
    // it; ties by index): the state passes dispatch the longest first.
    __shared__ int swork[1024];
    const int S = min(p.total_segs, 1024);
    __syncthreads();   // the offset tables above are complete
    for (int i = tid; i < S; i += 1024) {
      int lo = 0, hi = N - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (p.seg_off[mid] <= i) lo = mid; else hi = mid - 1;
      }
      const int ps = i - p.seg_off[lo], ch = p.chunk_off[lo + 1] - p.chunk_off[lo], L = p.seg_chunks;
      swork[i] = max(0, min(L, ch - ps * L)) + (ps > 0 ? min(p.warmup, ps * L) : 0);
    }
    __syncthreads();
    for (int i = tid; i < S; i += 1024) {
      const int wi = swork[i];
      int r = 0;
      for (int j = 0; j < S; ++j) r += (swork[j] > wi || (swork[j] == wi && j < i)) ? 1 : 0;
      p.seg_order[r] = i;
    }
  }
}

// Locates chunk c: sequence n, first token t0 and valid length; false if the
// device tables disagree with the grid (then the workgroup writes nothing).
__device__ __forceinline__ bool locate_chunk(const SeqTables& s, int c, int& n, int& t0, int& len) {
  if (c >= s.NTtot) return false;
  n = s.seq_of_chunk(c);
  t0 = s.cu_at(n) + (c - s.chunk_at(n)) * CH;
  len = min(CH, s.cu_at(n + 1) - t0);
  return len > 0 && t0 >= 0 && (long)t0 + len <= s.Ttot;
}

// --------------------------------------------------------------- k_intra --
// Persistent: each workgroup walks a contiguous range of (chunk, value head)
// items (value heads of one chunk adjacent, so the shared K tile is an L2
// hit) and loads the next item's K, V, g and beta into a second register set
// while the current one is computed.  Each wave owns one row block (16
// tokens) of A, W and U; "wave i" below means the owner of row block i.
// Per item:
//   1. K, V -> LDS with permuted columns (RowSlab); gate scan.
//   2. L = strict_lower(diag(b)(D * K K^T)) in fp32, ten lower 16x16 tiles
//      spread 3/2/3/2 over the waves; the diagonal of K K^T certifies
//      0 <= b |k|^2 <= 2 for the context-parallel warmup.
//   3. Inverse of the unit lower triangular I + L, blocked by 16: wave i
//      inverts its diagonal block by forward substitution, A_ii, and forms
//      M_ij = A_ii L_ij (j < i).  Since A_ij = -A_ii sum_{j<=m<i} L_im A_mj,
//        A_i,i-1 = -M_i,i-1 A_i-1,i-1
//        A_20 = -M_20 A_00 + M_21 T_10,         T_10 = M_10 A_00
//        A_31 = -M_31 A_11 + M_32 T_21,         T_21 = M_21 A_11
//        A_30 = -M_30 A_00 + M_31 T_10 - M_32 A_20
//      so each wave derives its whole row block from the shared M and A_ii
//      tiles, keeping intermediates in registers: a register tile enters a
//      product only as the right factor, whose accumulator layout already is
//      an MFMA B operand once the contraction index is permuted to match.
//   4. A' = A diag(b Gamma), A'' = A diag(b) in the working dtype, stored
//      transposed over the fp32 tiles.
//   5. W = A' K and U = A'' V: both operands are read with transposing LDS
//      loads, and each lane stores NT consecutive columns of its rows.
// Five workgroup barriers per item.
struct IntraItem {
  int c, h, hk, n, t0, len;
  bool ok;
};

// 16 x 16 fp32 tile products on V_MFMA_F32_16X16X4_F32 with the contraction
// index 4q + s at step s for lane group q.  The A operand (row t of X,
// columns 4q..4q+3) is one 16-byte LDS read; the B operand is a tile in
// accumulator layout (lane group q holds rows 4q..4q+3 of column t), which is
// where a product's result already is, or ld_acc() of an LDS tile.
template <int P>
__device__ __forceinline__ f32x4 ld_a(const float* X) {
  return *reinterpret_cast<const f32x4*>(X + (lane_id() & 15) * P + 4 * (lane_id() >> 4));
}
__device__ __forceinline__ f32x4 mm(f32x4 acc, f32x4 a, f32x4 b) {
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
  return acc;
}
// LDS tile -> accumulator layout, and back.
template <int P>
__device__ __forceinline__ f32x4 ld_acc(const float* X) {
  f32x4 a;
#pragma unroll
  for (int e = 0; e < 4; ++e) a[e] = X[acc_row(e) * P + acc_col()];
  return a;
}
template <int P>
__device__ __forceinline__ void st_acc(float* X, f32x4 a) {
#pragma unroll
  for (int e = 0; e < 4; ++e) X[acc_row(e) * P + acc_col()] = a[e];
}

// Lower tiles (i, j) of K K^T computed by the owner of row block w (n-th of kk_count(w)).
__device__ __forceinline__ int kk_count(int w) { return (w & 1) ? 2 : 3; }
__device__ __forceinline__ void kk_tile(int w, int n, int& i, int& j) {
  // w0: (0,0) (3,0) (3,1)   w1: (1,0) (1,1)   w2: (2,0) (2,1) (2,2)   w3: (3,2) (3,3)
  if (w == 0) { i = n == 0 ? 0 : 3; j = n == 0 ? 0 : n - 1; }
  else if (w == 1) { i = 1; j = n; }
  else if (w == 2) { i = 2; j = n; }
  else { i = 3; j = 2 + n; }
}

// (fp32 path; the bf16 path stores A diag(beta) rows instead: k_intra_w)
template <typename T, int KD>
__global__ __launch_bounds__(NTHR, 3) void k_intra(IntraParams p, int total_items, int per_wg, int nwg) {
  constexpr bool F32 = std::is_same<T, float>::value;
  constexpr int VD = KD;
  constexpr int NT = KD / 16;                 // column tiles of W and U
  constexpr int PK = Pitch<T, KD>::value;     // K / V rows (permuted columns)
  constexpr int PF = 68;                      // fp32 64-wide rows
  constexpr int PA = 68;                      // transposed A' / A''
  constexpr int SZ_K = CH * PK * (int)sizeof(T);
  constexpr int SZ_F = CH * PF * 4;
  constexpr int SZ_AT = 2 * CH * PA * (int)sizeof(T);
  constexpr int SZ_X = F32 ? SZ_AT : 0;       // fp32: A' / A'' cannot overlay the fp32 tiles
  static_assert(F32 || SZ_AT <= SZ_F, "A' and A'' must fit over the fp32 tiles");
  constexpr int NKV = 2;                      // staged row tiles: K and V
  __shared__ __align__(16) char smem[NKV * SZ_K + SZ_F + SZ_X];
  __shared__ float sG[CH], sB[CH];
  __shared__ int sFlag[NWAVE + 1];   // per-wave key-range flags, then the gate-sign flag
  T* sK = reinterpret_cast<T*>(smem);
  T* sV = reinterpret_cast<T*>(smem + (NKV - 1) * SZ_K);
  float* sF = reinterpret_cast<float*>(smem + NKV * SZ_K);
  T* sAw = reinterpret_cast<T*>(smem + NKV * SZ_K + (F32 ? SZ_F : 0));  // A'^T  [token j][token i]
  T* sAu = sAw + CH * PA;                                              // A''^T

  const SeqTables& s = p.s;
  const int x = xcd_remap(blockIdx.x, nwg);
  const int u0 = x * per_wg, u1 = min(total_items, u0 + per_wg);
  if (u0 >= u1) return;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  const int q = l >> 4, t = l & 15;
  // Row block of A, W, U owned by this wave.  The blocks differ in work (the
  // last has the longest inverse chain and contraction), so the assignment
  // rotates with the workgroup to spread the heavy one over the SIMDs.
  const int rb = (w + x) & 3;
  auto tile = [&](int i, int j) { return sF + 16 * i * PF + 16 * j; };

  auto locate = [&](int u, IntraItem& it) {
    it.ok = false;
    if (u >= u1) return;
    it.c = u / p.Hv;
    it.h = u - it.c * p.Hv;
    it.hk = it.h / (p.Hv / p.Hq);
    if (s.T_uniform > 0) {
      const int nc = (s.T_uniform + CH - 1) / CH;
      it.n = it.c / nc;
      const int cj = it.c - it.n * nc;
      it.t0 = it.n * s.T_uniform + cj * CH;
      it.len = min(CH, s.T_uniform - cj * CH);
      it.ok = it.c < s.NTtot && it.len > 0;
    } else {
      it.ok = locate_chunk(s, it.c, it.n, it.t0, it.len);
    }
  };
  // Loads of one item (an invalid item gets empty ranges: zeros, no traffic).
  auto fetch = [&](const IntraItem& it, RowSlab<T, KD>& rk, RowSlab<T, VD>& rv, float& gv, float& bv) {
    const int len = it.ok ? it.len : 0;
    const int t0 = it.ok ? it.t0 : 0;
    rk.load((const T*)p.k + ((long)t0 * p.Hq + it.hk) * KD, (long)p.Hq * KD, len);
    rv.load((const T*)p.v + ((long)t0 * p.Hv + it.h) * VD, (long)p.Hv * VD, len);
    const rsrc_t gr = make_rsrc(p.g + (long)t0 * p.Hv + it.h, (long)len * p.Hv * 4);
    const rsrc_t br = make_rsrc(p.beta + (long)t0 * p.Hv + it.h, (long)len * p.Hv * 4);
    gv = buf_load_f32(gr, (uint32_t)(l * p.Hv) * 4u);
    bv = buf_load_f32(br, (uint32_t)(l * p.Hv) * 4u);
  };

  auto run = [&](const IntraItem& it, RowSlab<T, KD>& rk, RowSlab<T, VD>& rv, float gvc, float bvc,
                 const IntraItem& nx, RowSlab<T, KD>& rkn, RowSlab<T, VD>& rvn, float& gvn, float& bvn) {
    const int t0 = it.t0, len = it.len, h = it.h;
    lds_barrier();  // the previous item is done with every LDS region
    if (w == 0) {
      const float gc = wave_inclusive_scan((l < len) ? gvc : 0.f);
      sG[l] = gc;
      sB[l] = (l < len) ? bvc : 0.f;
      // a token with g > 0 (or a NaN gate) voids the certificate
      const bool gpos = __builtin_amdgcn_ballot_w64(l < len && !(gvc <= 0.f)) != 0;
      if (l == 0) sFlag[NWAVE] = gpos ? 1 : 0;
      if (l < len) {
        p.gcum[(long)h * s.Ttot + t0 + l] = gc;
        if (p.g_cum_out) p.g_cum_out[(long)(t0 + l) * p.Hv + h] = gc;
      }
    }
    rk.template store_perm<PK>(sK);
    rv.template store_perm<PK>(sV);
    lds_barrier();
    fetch(nx, rkn, rvn, gvn, bvn);

    // 2. L tiles.
    {
      const int cnt = kk_count(rb);
      f32x4 acc[3];
      int ti[3], tj[3];
#pragma unroll
      for (int n = 0; n < 3; ++n) {
        acc[n] = zero4();
        kk_tile(rb, n, ti[n], tj[n]);
        if (n < cnt) mma_tile<T, KD, PK, 1, 1, PK>(acc[n], sK + 16 * ti[n] * PK, sK + 16 * tj[n] * PK);
      }
      int bad = 0;
#pragma unroll
      for (int n = 0; n < 3; ++n) {
        if (n < cnt) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 16 * ti[n] + acc_row(e), c = 16 * tj[n] + acc_col();
            float lv = 0.f;
            if (r > c) lv = sB[r] * __expf(sG[r] - sG[c]) * acc[n][e];
            if (r == c && r < len) {
              const float bn = sB[r] * acc[n][e];
              if (!(bn >= 0.f && bn <= 2.f)) bad = 1;
            }
            sF[r * PF + c] = lv;
          }
        }
      }
      const bool wave_bad = __builtin_amdgcn_ballot_w64(bad != 0) != 0;
      if (l == 0) sFlag[w] = wave_bad ? 1 : 0;
    }
    lds_barrier();
    if (tid == 0) {
      const int any_bad = sFlag[0] | sFlag[1] | sFlag[2] | sFlag[3] | sFlag[NWAVE];
      p.cert[(long)h * s.NTtot + it.c] = any_bad ? INFINITY : sG[len - 1];
    }

    // 3. Row block rb of A into registers a0..a3 (tile j), zero above the diagonal.
    f32x4 a0 = zero4(), a1 = zero4(), a2 = zero4(), a3 = zero4();
    if (p.A_in) {
      const float* src = p.A_in + ((long)t0 * p.Hv + h) * CH;
      const long rs = (long)p.Hv * CH;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rb + acc_row(e);
        if (r < len) {
          const float* row = src + (long)r * rs;
          if (0 <= rb && t < len) a0[e] = row[t];
          if (1 <= rb && 16 + t < len) a1[e] = row[16 + t];
          if (2 <= rb && 32 + t < len) a2[e] = row[32 + t];
          if (3 <= rb && 48 + t < len) a3[e] = row[48 + t];
        }
      }
    } else {
      // Diagonal block.  bf16: N = L_ii is nilpotent (N^16 = 0), so
      //   (I + N)^-1 = (I + N^8)(I + N^4)(I + N^2)(I - N),
      // applied right to left so that the running product is always the
      // right factor; N^2, N^4, N^8 pass through the tile itself.  Its fp32
      // rounding error (below 1e-3 even for nearly parallel keys) is under
      // the bf16 rounding that A' and A'' get next.  fp32: forward
      // substitution (lane l < 16 solves column l), exact to rounding.
      float* D = tile(rb, rb);
      f32x4 dg;
      if constexpr (F32) {
        if (l < 16) {
          float xs[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float acc = (r == l) ? 1.f : 0.f;
            const float* Lr = D + r * PF;
#pragma unroll
            for (int jj = 0; jj < r; ++jj) acc -= Lr[jj] * xs[jj];
            xs[r] = acc;
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) D[r * PF + l] = xs[r];
        }
        wave_sync();
        dg = ld_acc<PF>(D);
      } else {
        const f32x4 aN = ld_a<PF>(D), cN = ld_acc<PF>(D);
#pragma unroll
        for (int e = 0; e < 4; ++e) dg[e] = (acc_row(e) == acc_col() ? 1.f : 0.f) - cN[e];
        f32x4 pw = mm(zero4(), aN, cN);   // N^2
#pragma unroll
        for (int k = 0; k < 3; ++k) {     // N^(2^(k+1))
          wave_sync();
          st_acc<PF>(D, pw);
          wave_sync();
          const f32x4 ap = ld_a<PF>(D);
          dg = mm(dg, ap, dg);
          if (k < 2) pw = mm(zero4(), ap, pw);
        }
        wave_sync();
        st_acc<PF>(D, dg);
        wave_sync();
      }
      // M_ij = A_ii L_ij over L_ij.
      {
        const f32x4 aA = ld_a<PF>(D);
        for (int j = 0; j < rb; ++j) st_acc<PF>(tile(rb, j), mm(zero4(), aA, ld_acc<PF>(tile(rb, j))));
      }
      lds_barrier();
      if (rb == 0) {
        a0 = dg;
      } else if (rb == 1) {
        a0 = -mm(zero4(), ld_a<PF>(tile(1, 0)), ld_acc<PF>(tile(0, 0)));
        a1 = dg;
      } else if (rb == 2) {
        const f32x4 m10 = ld_a<PF>(tile(1, 0)), m20 = ld_a<PF>(tile(2, 0)), m21 = ld_a<PF>(tile(2, 1));
        const f32x4 d00 = ld_acc<PF>(tile(0, 0)), d11 = ld_acc<PF>(tile(1, 1));
        const f32x4 t10 = mm(zero4(), m10, d00);
        a0 = mm(-mm(zero4(), m20, d00), m21, t10);
        a1 = -mm(zero4(), m21, d11);
        a2 = dg;
      } else {
        const f32x4 m10 = ld_a<PF>(tile(1, 0)), m20 = ld_a<PF>(tile(2, 0)), m21 = ld_a<PF>(tile(2, 1));
        const f32x4 m30 = ld_a<PF>(tile(3, 0)), m31 = ld_a<PF>(tile(3, 1)), m32 = ld_a<PF>(tile(3, 2));
        const f32x4 d00 = ld_acc<PF>(tile(0, 0)), d11 = ld_acc<PF>(tile(1, 1)), d22 = ld_acc<PF>(tile(2, 2));
        const f32x4 t10 = mm(zero4(), m10, d00);
        const f32x4 t21 = mm(zero4(), m21, d11);
        const f32x4 a20 = mm(-mm(zero4(), m20, d00), m21, t10);
        a0 = mm(mm(-mm(zero4(), m30, d00), m31, t10), m32, -a20);
        a1 = mm(-mm(zero4(), m31, d11), m32, t21);
        a2 = -mm(zero4(), m32, d22);
        a3 = dg;
      }
    }
    if (p.A_ws || p.A_out || p.A_bf) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * rb + acc_row(e);
        if (r < len) {
          const float v4[4] = {a0[e], a1[e], a2[e], a3[e]};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (p.A_ws) p.A_ws[((long)h * s.Ttot + t0 + r) * CH + 16 * j + t] = v4[j];
            if (p.A_bf) ((bf16*)p.A_bf)[((long)h * s.Ttot + t0 + r) * CH + 16 * j + t] = from_f<bf16>(v4[j]);
            if (p.A_out) p.A_out[((long)(t0 + r) * p.Hv + h) * CH + 16 * j + t] = v4[j];
          }
        }
      }
    }

    // 4. A' and A'' (column scales b Gamma and b), transposed, over the fp32 tiles.
    float sw[4], su[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      su[j] = sB[16 * j + t];
      sw[j] = su[j] * __expf(sG[16 * j + t]);
    }
    lds_barrier();
    const int nks = F32 ? 4 * (rb + 1) : (rb + 2) / 2;  // contraction steps (A' is zero beyond 16(rb+1))
    const int ntile = F32 ? rb + 1 : 2 * nks;          // A' tiles the steps read
    {
      const f32x4 av[4] = {a0, a1, a2, a3};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j < ntile) {
          acc_store_t<T, PA>(sAw, 16 * rb, 16 * j, av[j], sw[j]);
          acc_store_t<T, PA>(sAu, 16 * rb, 16 * j, av[j], su[j]);
        }
      }
    }
    wave_sync();

    // 5. W = A' K, U = A'' V for row block rb.
    auto gemm_store = [&](const T* sAT, const T* sX, void* dst, int D) {
      f32x4 acc[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[j] = zero4();
      for (int ks = 0; ks < nks; ++ks) {
        if constexpr (F32) {
          const float a = sAT[(4 * ks + q) * PA + 16 * rb + t];
#pragma unroll
          for (int j = 0; j < NT; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, sX[(4 * ks + q) * PK + 16 * j + t], acc[j], 0, 0, 0);
        } else {
          const bf16x8 a = tr_frag(sAT + 32 * ks * PA + 16 * rb, PA);
#pragma unroll
          for (int j = 0; j < NT; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, tr_frag(sX + 32 * ks * PK + 16 * j, PK), acc[j], 0, 0, 0);
        }
      }
      const rsrc_t rr = make_rsrc((const T*)dst + ((long)h * s.Ttot + t0) * D, (long)len * D * (long)sizeof(T));
#pragma unroll
      for (int e = 0; e < 4; ++e)
        store_acc_row<T, NT>(rr, (uint32_t)(((16 * rb + acc_row(e)) * D + NT * t) * (int)sizeof(T)), acc, e);
    };
    gemm_store(sAw, sK, p.W, KD);
    gemm_store(sAu, sV, p.U, VD);
  };

  IntraItem cur, nxt;
  RowSlab<T, KD> rk0, rk1;
  RowSlab<T, VD> rv0, rv1;
  float g0 = 0.f, b0 = 0.f, g1 = 0.f, b1 = 0.f;
  locate(u0, cur);
  fetch(cur, rk0, rv0, g0, b0);
  for (int u = u0; u < u1; u += 2) {
    locate(u + 1, nxt);
    if (cur.ok) run(cur, rk0, rv0, g0, b0, nxt, rk1, rv1, g1, b1);
    else fetch(nxt, rk1, rv1, g1, b1);
    if (u + 1 >= u1) break;
    locate(u + 2, cur);
    if (nxt.ok) run(nxt, rk1, rv1, g1, b1, cur, rk0, rv0, g0, b0);
    else fetch(cur, rk0, rv0, g0, b0);
  }
}

// ------------------------------------------------------------- k_intra_w --
// The bf16 intra-chunk pass in A diag(beta) mode, one (chunk, value head)
// item per wave.  The items are independent and the whole 64 x 64 inverse of
// one item fits one wave's registers, so no workgroup barrier is needed: the
// sixteen waves a CU holds overlap each other's latencies (global loads, LDS
// round trips, the dependent fp32 MFMA chains of the inverse) instead of
// meeting at a barrier after every step.  Per item:
//   1. g, beta (lane = token) and the gate scan; K as bf16 MFMA fragments
//      straight from memory (lane (q, t) holds K[16i + t][32ks + 8q ..+8]),
//      which serve as both the A and the B operand of K K^T.
//   2. The ten lower 16 x 16 tiles of K K^T (fp32 accumulators), then L =
//      strict_lower(diag(b)(D * K K^T)) in place and the certificate check
//      0 <= b |k|^2 <= 2 on the diagonal.
//   3. The blocked inverse: diagonal blocks A_ii by forward substitution
//      (VALU, a lane per column), M_ij = A_ii L_ij, and the off-diagonal
//      blocks from M and the A_ii as in k_intra.  A product's left factor must
//      be in MFMA A layout (lane t holds row t): accumulator tiles get there
//      through a per-wave LDS tile (written by columns, read by rows).
//   4. A'' = A diag(b) rows in bf16 (and, with XA, A itself), staged as
//      rows in the wave's LDS area (over the tiles of step 3) and written
//      as 16-byte row pieces.
// XA: 0 A'' only; 1 also A in fp32 (A_ws and/or A_out, element stores); 2 also
// A in bf16 (A_bf, staged through LDS like A'').
template <int KD, int XA>
__global__ __launch_bounds__(NTHR, 4) void k_intra_w(IntraParams p, int total_items, int nwg) {
  constexpr int NKS = KD / 32;   // contraction steps of K K^T
  constexpr int TP = 20;         // row pitch of the per-wave fp32 tiles (16-byte rows)
  constexpr int NTT = 6;         // per-wave fp32 tiles
  constexpr int SP = CH + 8;      // row pitch (bf16) of the per-wave A'' staging rows
  constexpr int SCR = (CH * SP * 2 > NTT * 16 * TP * 4 ? CH * SP * 2 : NTT * 16 * TP * 4) / 4;
  __shared__ __align__(16) float sT[NWAVE][SCR];   // transposition tiles, later the A'' rows
  __shared__ __align__(16) float sGw[NWAVE][CH];
  __shared__ __align__(16) float sBw[NWAVE][CH];
  const SeqTables& s = p.s;
  const int w = wave_id(), l = lane_id(), q = l >> 4, t = l & 15;
  const int x = xcd_remap(blockIdx.x, nwg);
  if (x >= nwg) return;
  const int u = x * NWAVE + w;
  if (u >= total_items) return;
  const int c = u / p.Hv;
  const int h = u - c * p.Hv;
  const int hk = h / (p.Hv / p.Hq);
  int n, t0, len;
  if (s.T_uniform > 0) {
    const int nc = (s.T_uniform + CH - 1) / CH;
    n = c / nc;
    const int cj = c - n * nc;
    t0 = n * s.T_uniform + cj * CH;
    len = min(CH, s.T_uniform - cj * CH);
    if (c >= s.NTtot || len <= 0) return;
  } else if (!locate_chunk(s, c, n, t0, len)) {
    return;
  }
  float* sG = sGw[w];
  float* sB = sBw[w];
  auto tl = [&](int i) { return &sT[w][i * 16 * TP]; };
  bf16* sa = reinterpret_cast<bf16*>(&sT[w][0]);
  // accumulator tile -> rows of an LDS tile, and a row-layout (A operand) read
  auto st_t = [&](float* X, const f32x4& a) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 4; ++e) X[(4 * q + e) * TP + t] = a[e];
  };
  auto ld_t = [&](const float* X) __attribute__((always_inline)) {
    return *reinterpret_cast<const f32x4*>(X + t * TP + 4 * q);
  };

  // 1. loads (rows past the chunk read as zero)
  const rsrc_t gr = make_rsrc(p.g + (long)t0 * p.Hv + h, (long)len * p.Hv * 4);
  const rsrc_t br = make_rsrc(p.beta + (long)t0 * p.Hv + h, (long)len * p.Hv * 4);
  const float gv = buf_load_f32(gr, (uint32_t)(l * p.Hv) * 4u);
  const float bv = buf_load_f32(br, (uint32_t)(l * p.Hv) * 4u);
  const uint32_t krs = (uint32_t)(p.Hq * KD * 2);   // bytes between token rows of k
  const rsrc_t kr = make_rsrc((const bf16*)p.k + ((long)t0 * p.Hq + hk) * KD, (long)len * krs);
  bf16x8 kf[4][NKS];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const uint4 r = buf_load16(kr, (uint32_t)(16 * i + t) * krs + (uint32_t)(32 * ks + 8 * q) * 2u);
      __builtin_memcpy(&kf[i][ks], &r, 16);
    }
  const float gc = wave_inclusive_scan((l < len) ? gv : 0.f);
  sG[l] = gc;
  sB[l] = (l < len) ? bv : 0.f;
  if (l < len) {
    p.gcum[(long)h * s.Ttot + t0 + l] = gc;
    if (p.g_cum_out) p.g_cum_out[(long)(t0 + l) * p.Hv + h] = gc;
  }

  // 2. lower tiles of K K^T; tile (i, j) at index i(i+1)/2 + j
  f32x4 L[10];
#pragma unroll
  for (int m = 0; m < 10; ++m) L[m] = zero4();
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j <= i; ++j)
        L[i * (i + 1) / 2 + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[i][ks], kf[j][ks], L[i * (i + 1) / 2 + j], 0, 0, 0);
  wave_sync();   // sG, sB visible to the whole wave
  int bad = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x4 grow = *reinterpret_cast<const f32x4*>(sG + 16 * i + 4 * q);
    const f32x4 brow = *reinterpret_cast<const f32x4*>(sB + 16 * i + 4 * q);
#pragma unroll
    for (int j = 0; j <= i; ++j) {
      const float gcol = sG[16 * j + t];
      f32x4& a = L[i * (i + 1) / 2 + j];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * i + 4 * q + e, cc = 16 * j + t;
        if (i == j) {   // diagonal of K K^T: branch-free range check of b |k|^2
          const float bn = brow[e] * a[e];
          bad |= (r == cc && r < len && !(bn >= 0.f && bn <= 2.f)) ? 1 : 0;
        }
        const float lv = brow[e] * __expf(grow[e] - gcol) * a[e];
        a[e] = (i > j || r > cc) ? lv : 0.f;
      }
    }
  }
  // a token with g > 0 (or a NaN gate) also voids the certificate: the
  // contraction bound of the warmup error needs every gate in (0, 1]
  bad |= (l < len && !(gv <= 0.f)) ? 1 : 0;
  const bool any_bad = __builtin_amdgcn_ballot_w64(bad != 0) != 0;
  if (l == 0) p.cert[(long)h * s.NTtot + c] = any_bad ? INFINITY : sG[len - 1];

  // 4. (16 x 16 blocks of A emitted once the transposition tiles are no
  // longer needed) A'' = A diag(b) staged as bf16 rows in LDS, then written
  // as 16-byte row pieces (zero above the diagonal blocks); A itself when
  // asked for.
  float su[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) su[j] = sB[16 * j + t];
  const rsrc_t ar = make_rsrc((bf16*)p.Au + ((long)h * s.Ttot + t0) * CH, apack_bytes(len));   // compact rows
  // A itself (XA): fp32 or bf16 head-major rows, or fp32 token-major rows
  // (a null pointer gets an empty range: its stores are dropped)
  const long hrow = ((long)h * s.Ttot + t0) * CH;
  const rsrc_t xw = make_rsrc(p.A_ws ? p.A_ws + hrow : nullptr, p.A_ws ? (long)len * CH * 4 : 0);
  const rsrc_t xb = make_rsrc(p.A_bf ? (bf16*)p.A_bf + hrow : nullptr, p.A_bf ? (long)len * CH * 2 : 0);
  const rsrc_t xo = make_rsrc(p.A_out ? p.A_out + ((long)t0 * p.Hv + h) * CH : nullptr,
                              p.A_out ? (long)len * p.Hv * CH * 4 : 0);
  auto store_a = [&](int i, int j, const f32x4& v) __attribute__((always_inline)) {
    if constexpr (XA == 1) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t r = (uint32_t)(16 * i + 4 * q + e), cc = (uint32_t)(16 * j + t);
        buf_store4(xw, (r * CH + cc) * 4u, __float_as_uint(v[e]));
        buf_store4(xo, (r * (uint32_t)(p.Hv * CH) + cc) * 4u, __float_as_uint(v[e]));
      }
    }
  };
  // the blocks above the diagonal of A are zero
#pragma unroll
  for (int i = 0; i < 3; ++i)
#pragma unroll
    for (int j = i + 1; j < 4; ++j) store_a(i, j, zero4());
  // Staging: without a bf16 A the A'' rows of all 64 tokens; with it, A'' and
  // A rows of one 32-token half at a time (sa: A'', sa + 32 SP: A).
  constexpr bool two = XA == 2;
  auto emit = [&](int i, int j, f32x4 v) __attribute__((always_inline)) {
    store_a(i, j, v);
#pragma unroll
    for (int e = 0; e < 4; e += 2) {   // two rows per conversion
      const int r = 16 * i + 4 * q + e;
      const bf16x2 av = __builtin_convertvector((f32x2){v[e] * su[j], v[e + 1] * su[j]}, bf16x2);
      const int ra = two ? (r & 31) : r;
      sa[ra * SP + 16 * j + t] = av[0];
      sa[(ra + 1) * SP + 16 * j + t] = av[1];
      if (two) {
        const bf16x2 au = __builtin_convertvector((f32x2){v[e], v[e + 1]}, bf16x2);
        sa[(32 + ra) * SP + 16 * j + t] = au[0];
        sa[(33 + ra) * SP + 16 * j + t] = au[1];
      }
    }
  };
  // 16-byte row pieces from the staging rows to memory: A'' as compact rows
  // (the pieces above the diagonal blocks get an out-of-range offset, so
  // their stores are dropped), A with zeros there; half < 0: all 64 A''
  // rows, else one half of A'' and A.
  auto flush = [&](int half) __attribute__((always_inline)) {
    wave_sync();
    const int pc = l & 7;   // 16-byte piece of a row: columns 8pc .. 8pc + 7
    if (half < 0) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int r = (l >> 3) + 8 * k;
        const uint4 v = *reinterpret_cast<const uint4*>(sa + r * SP + 8 * pc);
        buf_store16(ar, apack_src(r, pc), v);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int rl = (l >> 3) + 8 * k, r = 32 * half + rl;
        const uint4 v = *reinterpret_cast<const uint4*>(sa + rl * SP + 8 * pc);
        uint4 u = *reinterpret_cast<const uint4*>(sa + (32 + rl) * SP + 8 * pc);
        if (pc >= 2 * ((r >> 4) + 1)) u = make_uint4(0u, 0u, 0u, 0u);
        buf_store16(ar, apack_src(r, pc), v);
        buf_store16(xb, (uint32_t)(r * CH + 8 * pc) * 2u, u);
      }
      wave_sync();   // the half's rows are read before the next half is staged
    }
  };

  // 3. A = (I + L)^-1 by 16 x 16 blocks.
  if (p.A_in) {
    const float* src = p.A_in + ((long)t0 * p.Hv + h) * CH;
    const long rs = (long)p.Hv * CH;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j <= i; ++j) {
        f32x4 v = zero4();
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * i + 4 * q + e;
          if (r < len && 16 * j + t < len) v[e] = src[(long)r * rs + 16 * j + t];
        }
        emit(i, j, v);
      }
      if (i == 1 && two) flush(0);
    }
    flush(two ? 1 : -1);
    return;
  }
  // Diagonal blocks by forward substitution on the VALU: lane group b
  // solves column t of (I + N_b)^-1, N_b = L_bb, reading the rows of N_b as
  // LDS broadcasts; the solved column is written back as row t of A_bb^T,
  // from which both layouts of A_bb are single reads.
#pragma unroll
  for (int i = 0; i < 4; ++i) st_t(tl(i), L[i * (i + 1) / 2 + i]);
  wave_sync();
  float xs[16];
  {
    const float* nb = tl(q);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = (r == t) ? 1.f : 0.f;
#pragma unroll
      for (int j4 = 0; j4 < r; j4 += 4) {
        const f32x4 nr = *reinterpret_cast<const f32x4*>(nb + r * TP + j4);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          if (j4 + jj < r) acc -= nr[jj] * xs[j4 + jj];
      }
      xs[r] = acc;
    }
  }
  wave_sync();
  {
    float* yb = tl(q);
#pragma unroll
    for (int r4 = 0; r4 < 16; r4 += 4)
      *reinterpret_cast<f32x4*>(yb + t * TP + r4) = f32x4{xs[r4], xs[r4 + 1], xs[r4 + 2], xs[r4 + 3]};
  }
  wave_sync();
  f32x4 dg[4], da[4];   // A_ii in accumulator layout and (i >= 1) in A layout
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    dg[i] = ld_t(tl(i));
#pragma unroll
    for (int e = 0; e < 4; ++e) da[i][e] = (i > 0) ? tl(i)[(4 * q + e) * TP + t] : 0.f;
  }
  // M_ij = A_ii L_ij (j < i), then into A layout
  {
    f32x4 mc[6];   // (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
    mc[0] = mm(zero4(), da[1], L[1]);
    mc[1] = mm(zero4(), da[2], L[3]);
    mc[2] = mm(zero4(), da[2], L[4]);
    mc[3] = mm(zero4(), da[3], L[6]);
    mc[4] = mm(zero4(), da[3], L[7]);
    mc[5] = mm(zero4(), da[3], L[8]);
    wave_sync();
#pragma unroll
    for (int m = 0; m < 6; ++m) st_t(tl(m), mc[m]);
    wave_sync();
  }
  const f32x4 m10 = ld_t(tl(0)), m20 = ld_t(tl(1)), m21 = ld_t(tl(2));
  const f32x4 m30 = ld_t(tl(3)), m31 = ld_t(tl(4)), m32 = ld_t(tl(5));
  wave_sync();   // the tiles are free: the A'' rows are staged over them
  emit(0, 0, dg[0]);
  emit(1, 1, dg[1]);
  const f32x4 t10 = mm(zero4(), m10, dg[0]);
  emit(1, 0, -t10);
  if (two) flush(0);
  emit(2, 2, dg[2]);
  emit(3, 3, dg[3]);
  const f32x4 t21 = mm(zero4(), m21, dg[1]);
  emit(2, 1, -t21);
  emit(3, 2, -mm(zero4(), m32, dg[2]));
  const f32x4 a20 = mm(-mm(zero4(), m20, dg[0]), m21, t10);
  emit(2, 0, a20);
  emit(3, 1, mm(-mm(zero4(), m31, dg[1]), m32, t21));
  emit(3, 0, mm(mm(-mm(zero4(), m30, dg[0]), m31, t10), m32, -a20));
  flush(two ? 1 : -1);
}

// --------------------------------------------------------------- k_state --
// One workgroup per (sequence, value head, V block, CP segment), serial over
// the segment's chunks.  h (K x BV) stays in fp32 MFMA accumulators; the next
// chunk's W, K, U rows are fetched into registers while the current one runs.
// Used by the backward to recompute every chunk's entry state: hbuf receives
// [K][V] per chunk and vnew the token rows [Ttot][V] (the layouts the gradient
// kernels read).  ROWS = false keeps the transposed per-chunk layouts.
template <typename T, int KD, int BV, bool ROWS>
__global__ __launch_bounds__(NTHR) void k_state(StateParams p, int total_items) {
  constexpr int VD = KD;
  constexpr int PK = Pitch<T, KD>::value;
  constexpr int PU = Pitch<T, BV>::value;
  constexpr int PT = Pitch<T, CH>::value;
  constexpr int NCB = BV / 16;
  constexpr int NTILE = (KD / 16) * NCB;
  constexpr int TPW = NTILE / NWAVE;
  static_assert(NTILE % NWAVE == 0, "state tiles must split evenly over the waves");
  __shared__ __align__(16) T sW[CH * PK];
  __shared__ __align__(16) T sKdT[KD * PT];
  __shared__ __align__(16) T sU[CH * PU];
  __shared__ __align__(16) T shT[BV * PK];
  __shared__ __align__(16) T sVt[BV * PT];
  __shared__ __align__(16) T sRows[ROWS ? KD * PU + CH * PU : 8];  // [K][BV] state, then [64][BV] Vnew
  T* sHr = sRows;
  T* sVr = sRows + (ROWS ? KD * PU : 0);

  const SeqTables& s = p.s;
  const int u = xcd_remap(blockIdx.x, total_items);
  if (u >= total_items) return;
  const int vb = u % p.nvb;
  const int h = (u / p.nvb) % p.Hv;
  const int item = u / (p.nvb * p.Hv);
  const int n = s.seq_of_seg(item);
  const int pseg = item - s.seg_at(n);
  const int nseg = s.seg_at(n + 1) - s.seg_at(n);
  const int c0 = s.chunk_at(n);
  const int nch = s.chunk_at(n + 1) - c0;
  if (pseg < 0 || pseg >= nseg || c0 < 0 || c0 + nch > s.NTtot) return;
  const int L = p.seg_chunks;
  const int hk = h / (p.Hv / p.Hq);
  const int w = wave_id();

  // A head is certified when every warmup window's gate mass is small enough
  // (all segments of the head evaluate the same test, so they agree).
  const bool certified = head_certified(p.cert + (long)h * s.NTtot + c0, nseg, nch, L, p.warmup, p.log_eps, false);
  int cstart, cbeg, cend;
  bool write_final;
  if (!certified) {
    if (pseg != 0) return;             // segment 0 runs the whole head serially
    cstart = 0; cbeg = 0; cend = nch; write_final = true;
  } else {
    cbeg = pseg * L;
    cend = min(cbeg + L, nch);
    cstart = (pseg == 0) ? 0 : max(0, cbeg - p.warmup);
    write_final = (pseg == nseg - 1);
  }

  f32x4 hacc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int ti = w * TPW + i, rb = ti / NCB, cb = ti % NCB;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int d = 16 * rb + acc_row(e), v = vb * BV + 16 * cb + acc_col();
      hacc[i][e] = (cstart == 0 && p.h0) ? p.h0[(((long)n * p.Hv + h) * KD + d) * VD + v] : 0.f;
    }
  }

  TileRegs<T, CH, KD> rw;
  TileCols<T, KD> rk;
  TileRegs<T, CH, BV> ru;
  float gam = 0.f;
  float glast_next = 0.f;
  auto prefetch = [&](int jc) {  // unconditional; empty range past the segment
    const bool valid = jc < cend;
    const int t0 = s.cu_at(n) + min(jc, cend - 1) * CH;
    const int len = valid ? min(CH, s.cu_at(n + 1) - t0) : 0;
    rw.load((const T*)p.W + ((long)h * s.Ttot + t0) * KD, KD, len);
    rk.load((const T*)p.k + ((long)t0 * p.Hq + hk) * KD, (long)p.Hq * KD, len);
    ru.load((const T*)p.U + ((long)h * s.Ttot + t0) * VD + vb * BV, VD, len);
    const rsrc_t gr = make_rsrc(p.gcum + (long)h * s.Ttot + t0, (long)len * 4);
    const float gv = buf_load_f32(gr, (uint32_t)lane_id() * 4u);
    gam = (lane_id() < len) ? gv : 0.f;
    glast_next = buf_load_f32(gr, (uint32_t)(len - 1) * 4u);
  };
  if (cstart < cend) prefetch(cstart);

  for (int jc = cstart; jc < cend; ++jc) {
    const int gc = c0 + jc;
    const int t0 = s.cu_at(n) + jc * CH;
    const int len = min(CH, s.cu_at(n + 1) - t0);
    const bool warm = jc < cbeg;
    const float glast = glast_next;
    rw.template store<PK>(sW);
    ru.template store<PU>(sU);
    // transposed, decayed K: sKdT[d][t] = e^{gamma_n - gamma_t} k_t[d]
    rk.template store_t<PT>(sKdT, (lane_id() < len) ? __expf(glast - gam) : 0.f);
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int ti = w * TPW + i, rb = ti / NCB, cb = ti % NCB;
      acc_store_t<T, PK>(shT, 16 * rb, 16 * cb, hacc[i]);
      if constexpr (ROWS) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sHr[(16 * rb + acc_row(e)) * PU + 16 * cb + acc_col()] = from_f<T>(hacc[i][e]);
      }
    }
    lds_barrier();
    prefetch(jc + 1);
    if (!warm && p.hbuf) {
      if constexpr (ROWS)
        store_rows<T, KD, BV, PU>((T*)p.hbuf + ((long)h * s.NTtot + gc) * KD * VD + vb * BV, VD, sHr, KD);
      else
        store_rows<T, BV, KD, PK>((T*)p.hbuf + (((long)h * s.NTtot + gc) * VD + vb * BV) * KD, KD, shT, BV);
    }

    {  // Vnew = U - W h, staged transposed (tokens contiguous)
      f32x4 acc[NCB];
#pragma unroll
      for (int j = 0; j < NCB; ++j) acc[j] = zero4();
      mma_row<T, KD, NCB, PK, 1, 1, PK>(acc, sW + 16 * w * PK, shT);
#pragma unroll
      for (int j = 0; j < NCB; ++j) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[j][e] = to_f(sU[(16 * w + acc_row(e)) * PU + 16 * j + acc_col()]) - acc[j][e];
        acc_store_t<T, PT>(sVt, 16 * w, 16 * j, acc[j]);
        if constexpr (ROWS) {
#pragma unroll
          for (int e = 0; e < 4; ++e) sVr[(16 * w + acc_row(e)) * PU + 16 * j + acc_col()] = from_f<T>(acc[j][e]);
        }
      }
    }
    lds_barrier();
    if (!warm) {
      if constexpr (ROWS)
        store_rows<T, CH, BV, PU>((T*)p.vnew + ((long)h * s.Ttot + t0) * VD + vb * BV, VD, sVr, len);
      else
        store_rows<T, BV, CH, PT>((T*)p.vnew + (((long)h * s.NTtot + gc) * VD + vb * BV) * CH, CH, sVt, BV);
    }

    const float dlast = __expf(glast);
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int ti = w * TPW + i, rb = ti / NCB, cb = ti % NCB;
      hacc[i] *= dlast;
      mma_tile<T, CH, PT, 1, 1, PT>(hacc[i], sKdT + 16 * rb * PT, sVt + 16 * cb * PT);
    }
    lds_barrier();
  }

  if (write_final && p.ht) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int ti = w * TPW + i, rb = ti / NCB, cb = ti % NCB;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = 16 * rb + acc_row(e), v = vb * BV + 16 * cb + acc_col();
        p.ht[(((long)n * p.Hv + h) * KD + d) * VD + v] = hacc[i][e];
      }
    }
  }
}

// ---------------------------------------------------------------- k_fused --
// The serial chunk recurrence fused with the output (the pages' second fused
// forward kernel: FlashQLA curated summary, section
// "平衡解決方案：雙核心融合與自動CP"): one 8-wave workgroup per (sequence,
// value head, CP segment).  Wave w owns 16 state columns over all K rows, in
// fp32 accumulators, so the recurrence needs no data from other waves:
//   Vnew = U - W h            (h, as accumulators, is the MFMA B operand)
//   h'   = Gamma_n h + K^T (d * Vnew),  d_t = e^{gamma_n - gamma_t}
//                             (Vnew, as accumulators, is the B operand; K
//                             is read with transposing LDS loads)
//   O    = s Gamma (Q h) + P Vnew,  P = s lower(D * Q K^T)
// The chunk inputs W, Q, K, U and the gate cumsums are copied from global
// memory straight into LDS (buffer loads with the LDS destination bit),
// double-buffered: the next chunk's copy is issued during a chunk and
// waited for at its end, so it overlaps the chunk and costs no registers.
// Every staged tile is its own LDS array and the chunk loop is unrolled by
// two, so each chunk reads one fixed set of arrays and copies into the
// other: the compiler then sees that the reads cannot alias the copies in
// flight and does not wait for them before every LDS read.  Staged tiles are unpadded with the 16-byte pieces of each row
// XOR-swizzled (row-dependent), which keeps the 8-byte fragment reads and
// the transposing reads free of bank conflicts.  P tiles are shared (one or
// two per wave); the bf16 output is staged in LDS and written as full rows.
// Two workgroup barriers per chunk.  Two waves per SIMD hide each other's
// LDS and MFMA latencies.
// Segment transitions (MODE 2, heads that fail the warmup certificate):
// the map from a segment's start state to its end state is affine,
// h_out = M h_in + b, so one workgroup per (segment, part) runs the segment's
// chunks without output from h = I with U taken as zero (part 0: M, from the
// second segment on) or from h = 0, the initial state for the first segment,
// with U (part 1: b), and stores the end state.  k_segscan chains them into
// exact start states, from which the output pass then runs every segment.
// Row numbering: state tile rb, lane group g, element e holds K row
// 32(rb/2) + 8g + 4(rb%2) + e, so the two tiles of a 32-row contraction step
// give a lane K rows 32ks + 8g .. +7, and the W and Q fragments that match
// them are single 16-byte LDS reads.  P is stored with its token columns
// permuted the same way (32-token block, group g, half hh: column
// 32ks + 16hh + 4g + e at position 32ks + 8g + 4hh + e) for P Vnew.
template <typename T>
struct FusedBufs {   // one buffer of staged chunk inputs
  T *W, *Q, *K, *U;
  float *G, *D;      // gate cumsums; per-row factors {e^{gamma_n - gamma_t}, s e^{gamma_t}}
};

// MODE: 0 the output pass, 1 the backward's states pass, 2 the forward's
// segment transitions, 3 the backward's, 4 the output pass with Vnew split
// into two bf16 terms in its products (separate instantiations, so each
// keeps only its own paths).
template <typename T, int KD, int MODE>
__global__ __launch_bounds__(FNT) void k_fused(FusedParams p, int total_items) {
  constexpr bool TRANS = MODE == 2 || MODE == 3;
  // Vnew as hi + lo, two bf16 terms (hi = bf16(x), lo = bf16(x - hi)), in
  // both products that take it as an MFMA operand (P Vnew and the state
  // update): an error of about 2^-16 of |Vnew| instead of the 2^-9 of one
  // bf16 rounding, for strongly coupled keys (two MFMAs per product).
  constexpr bool SPLITV = MODE == 4;
  constexpr bool F32 = std::is_same<T, float>::value;
  constexpr int VD = KD;
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int NCH = KD / VEC;                    // 16-byte pieces per staged row
  constexpr int PP = Pitch<T, CH>::value;
  constexpr int TE = CH * KD;                      // elements per staged tile
  constexpr int NKB = KD / 16, NCB = VD / 16;
  constexpr int NWV = NCB < FNW ? NCB : FNW;       // waves owning state columns
  constexpr int CBW = NCB / NWV;                   // column tiles per owning wave
  static_assert(CBW == 1, "one column tile per wave");
  // bf16 passes stage A'' = A diag(beta) (64 x 64) and V instead of W and U,
  // and form Vnew = A''(V - Gamma * K h) themselves.
  constexpr bool AP = !F32;
  constexpr int TW = AP ? CH * CH : TE;
  __shared__ __align__(16) T sW0[TW], sQ0[TE], sK0[TE], sU0[TE], sW1[TW], sQ1[TE], sK1[TE], sU1[TE];
  // P: bf16 as a swizzled 64-wide tile (16-byte fragment reads without bank
  // conflicts), fp32 row-padded
  constexpr int PSZ = F32 ? CH * PP : CH * CH;
  __shared__ __align__(16) T sP[PSZ];
  __shared__ __align__(16) T sO[F32 ? 8 : TE];     // bf16 output rows (fp32 stores directly)
  __shared__ __align__(16) float sG0[CH], sG1[CH], sD0[3 * CH], sD1[3 * CH];
  if (p.Hq < 0) {  // never taken: an ordinary store keeps the copy-only arrays from being folded away
    const T z = from_f<T>(0.f);
    sW0[threadIdx.x] = z; sQ0[threadIdx.x] = z; sK0[threadIdx.x] = z; sU0[threadIdx.x] = z;
    sW1[threadIdx.x] = z; sQ1[threadIdx.x] = z; sK1[threadIdx.x] = z; sU1[threadIdx.x] = z;
    sG0[threadIdx.x & 63] = 0.f; sG1[threadIdx.x & 63] = 0.f;
  }
  auto bufs = [&](auto bc) __attribute__((always_inline)) {
    if constexpr (decltype(bc)::value == 0) return FusedBufs<T>{sW0, sQ0, sK0, sU0, sG0, sD0};
    else return FusedBufs<T>{sW1, sQ1, sK1, sU1, sG1, sD1};
  };
  // element offset of (row, col) in a staged tile
  auto tix = [](int r, int c) { return (r * NCH + ((c / VEC) ^ stage_swz<NCH>(r))) * VEC + (c % VEC); };

  const SeqTables& s = p.s;
  int h, item2;
  if (!TRANS && s.seg_order) {
    // Unequal segments: groups of the G value heads that share q and k, in
    // decreasing segment work, go round-robin over the 8 XCDs (block b runs
    // on XCD b mod 8); a group's heads take consecutive slots of one XCD.
    const int G = p.Hv / p.Hq;
    const int x = (int)blockIdx.x & 7, pos = (int)blockIdx.x >> 3;
    const int kg = (pos / G) * 8 + x;
    if (kg >= p.total_segs * p.Hq) return;
    const int r = kg / p.Hq;
    item2 = s.seg_order[r];
    h = (kg - r * p.Hq) * G + pos % G;
  } else {
    const int u = xcd_remap(blockIdx.x, total_items);
    if (u >= total_items) return;
    h = u % p.Hv;
    item2 = u / p.Hv;
  }
  const int part = TRANS ? (item2 & 1) : 1;   // transition pass: 0 M, 1 b
  const int item = TRANS ? (item2 >> 1) : item2;
  const int n = s.seq_of_seg(item);
  const int pseg = item - s.seg_at(n);
  const int nseg = s.seg_at(n + 1) - s.seg_at(n);
  const int c0 = s.chunk_at(n);
  const int nch = s.chunk_at(n + 1) - c0;
  if (pseg < 0 || pseg >= nseg || c0 < 0 || c0 + nch > s.NTtot) return;
  const int seq0 = s.cu_at(n), seq1 = s.cu_at(n + 1);   // token range of the sequence
  const int L = p.seg_chunks;
  const int hk = h / (p.Hv / p.Hq);
  const int w = wave_id(), l = lane_id(), q = l >> 4, t = l & 15;
  const bool owner = NWV == FNW || w < NWV;   // a constant when every wave owns columns
  auto vcol = [&](int cb) { return CBW == 2 ? 32 * w + 2 * t + cb : 16 * w + t; };

  const float* hcert = p.cert + (long)h * s.NTtot + c0;
  const float wpre = TRANS ? 0.f : warmup_first(hcert, pseg * L - 1, -1, pseg * L, p.warmup);
  // The head's certificate: the transition pass evaluates it and records
  // the decision for the later passes of the same call, which read it.
  bool certified;
  if (!TRANS && p.hflag) {
    certified = p.hflag[(long)n * p.Hv + h] != 0;
  } else {
    certified = head_certified(hcert, nseg, nch, L, p.warmup, p.log_eps, p.rev_cert != 0);
    if (TRANS && p.hflag && pseg == 0 && part == 0 && threadIdx.x == 0) p.hflag[(long)n * p.Hv + h] = certified ? 1 : 0;
  }
  const int gseg = s.seg_at(n) + pseg;          // global segment index
  const bool exact = !certified && p.hstart != nullptr;
  int cstart, cbeg, cend;
  bool write_final;
  if (TRANS) {   // uncertified heads only; the last segment's map is not needed
    if (certified || pseg == nseg - 1 || (part == 0 && pseg == 0)) return;
    cbeg = cstart = pseg * L;
    cend = min(cbeg + L, nch);
    write_final = false;
  } else if (certified) {
    cbeg = pseg * L;
    cend = min(cbeg + L, nch);
    const int wu = short_warmup(hcert, cbeg - 1, -1, cbeg, p.warmup, p.log_eps, wpre);
    cstart = (pseg == 0) ? 0 : max(0, cbeg - wu);
    write_final = (pseg == nseg - 1);
  } else if (exact) {
    cbeg = cstart = pseg * L;
    cend = min(cbeg + L, nch);
    write_final = (pseg == nseg - 1);
  } else {
    if (pseg != 0) return;             // segment 0 runs the whole head serially
    cstart = 0; cbeg = 0; cend = nch; write_final = true;
  }
  const bool no_u = TRANS && part == 0;         // M: the segment's map with U = 0
  const bool st_mode = MODE == 1;   // backward recompute: states, no output

  const long hbase = ((long)n * p.Hv + h) * KD * VD;
  auto krow = [&](int rb, int e) { return 32 * (rb >> 1) + 8 * q + 4 * (rb & 1) + e; };
  // Initial state: h0 at a sequence start, an exact start state, the identity
  // (transition part 0) or zero.
  const float* hinit = nullptr;
  if (TRANS) {
    if (part == 1 && pseg == 0 && p.h0) hinit = p.h0 + hbase;
  } else if (cstart == 0) {
    if (p.h0) hinit = p.h0 + hbase;
  } else if (exact) {
    hinit = p.hstart + ((long)h * p.total_segs + gseg) * KD * VD;
  }
  // One branch around all the loads, so that they are issued together.
  f32x4 hs[NKB][CBW];
#pragma unroll
  for (int rb = 0; rb < NKB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CBW; ++cb) hs[rb][cb] = zero4();
  if (owner && hinit) {
#pragma unroll
    for (int rb = 0; rb < NKB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CBW; ++cb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          hs[rb][cb][e] = hinit[(long)(F32 ? 16 * rb + acc_row(e) : krow(rb, e)) * VD + vcol(cb)];
  }
  if (TRANS && no_u && owner) {
#pragma unroll
    for (int rb = 0; rb < NKB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CBW; ++cb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          hs[rb][cb][e] = ((F32 ? 16 * rb + acc_row(e) : krow(rb, e)) == vcol(cb)) ? 1.f : 0.f;
  }

  // Copies of chunk jc's tiles into buffer b (rows past the chunk read as
  // zero), in four parts (0 W, 1 U, 2 K, 3 Q and the gate cumsums); the
  // chunk loop issues W and U first and the rest after the P tiles, so that
  // no wave stalls long on a full memory queue.  The per-lane byte offsets within a tile do not
  // depend on the chunk.
  constexpr int NCP = (NCH + FNW - 1) / FNW;   // copy instructions per wave and tile
  uint32_t off_wu[NCP], off_qk[NCP], off_v[NCP], off_a[1];
#pragma unroll
  for (int j = 0; j < NCP; ++j) {
    const int i = w + FNW * j;
    const int pidx = 64 * i + l;
    const int r = pidx / NCH, c = (pidx % NCH) ^ stage_swz<NCH>(r);
    off_wu[j] = (uint32_t)(r * KD * (int)sizeof(T) + c * 16);
    off_qk[j] = (uint32_t)(r * p.Hq * KD * (int)sizeof(T) + c * 16);
    off_v[j] = (uint32_t)(r * p.Hv * VD * (int)sizeof(T) + c * 16);
  }
  {  // the 64-wide A'' tile: eight 1 KB blocks, one per wave, from compact rows
    const int pidx = 64 * w + l;
    const int r = pidx >> 3, c = (pidx & 7) ^ stage_swz<8>(r);
    off_a[0] = apack_src(r, c);
  }
  auto tix8 = [](int r, int c) { return (r * 8 + ((c >> 3) ^ stage_swz<8>(r))) * 8 + (c & 7); };
  auto copy_part = [&](int jc, auto bc, int piece) __attribute__((always_inline)) {
    const FusedBufs<T> bf = bufs(bc);
    const int t0 = seq0 + jc * CH;
    const int len = min(CH, seq1 - t0);
    const long wbytes = (long)len * KD * (long)sizeof(T), qbytes = wbytes * p.Hq;
    if constexpr (AP) {
      if (piece == 0)
        lds_copy_tile<1, 8, FNW, 8, true>(bf.W, rsrc_words((const T*)p.Au + ((long)h * s.Ttot + t0) * CH, apack_bytes(len)), off_a, w);
      if (piece == 1 && !no_u)
        lds_copy_tile<NCP, NCH, FNW, VEC, true>(bf.U, rsrc_words((const T*)p.v + ((long)t0 * p.Hv + h) * VD, wbytes * p.Hv), off_v, w);
    } else {
      if (piece == 0)
        lds_copy_tile<NCP, NCH, FNW, VEC>(bf.W, rsrc_words((const T*)p.W + ((long)h * s.Ttot + t0) * KD, wbytes), off_wu, w);
      if (piece == 1 && !no_u)
        lds_copy_tile<NCP, NCH, FNW, VEC>(bf.U, rsrc_words((const T*)p.U + ((long)h * s.Ttot + t0) * VD, wbytes), off_wu, w);
    }
    if (piece == 2)
      lds_copy_tile<NCP, NCH, FNW, VEC>(bf.K, rsrc_words((const T*)p.k + ((long)t0 * p.Hq + hk) * KD, qbytes), off_qk, w);
    if (piece == 3) {
      if (jc >= cbeg && !TRANS && !st_mode)
        lds_copy_tile<NCP, NCH, FNW, VEC>(bf.Q, rsrc_words((const T*)p.q + ((long)t0 * p.Hq + hk) * KD, qbytes), off_qk, w);
      if (w == 0) {
        const i32x4v gr = rsrc_words(p.gcum + (long)h * s.Ttot + t0, (long)len * 4);
        lds_copy4(gr, (uint32_t)l * 4u, lds_addr(bf.G));
      }
    }
  };
  auto copy_chunk = [&](int jc, auto bc) __attribute__((always_inline)) {
#pragma unroll
    for (int piece = 0; piece < 4; ++piece) copy_part(jc, bc, piece);
  };
  // Waits for this wave's copies; wave 0 (which copied the gate cumsums of
  // chunk jn into buffer bn) then derives that chunk's per-row factors; the
  // barrier publishes everything.
  auto wait_copies = [&](int jn, auto bc) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0);   // vmcnt = 0 (the LDS copies), expcnt = 0, lgkmcnt = 0
    if (w == 0 && jn < cend) {
      const FusedBufs<T> bf = bufs(bc);
      const int tn = seq0 + jn * CH;
      const int ln = min(CH, seq1 - tn);
      const float gl = bf.G[max(ln, 1) - 1], gv = bf.G[l];
      bf.D[l] = (l < ln) ? __expf(gl - gv) : 0.f;
      bf.D[CH + l] = p.scale * __expf(gv);
      bf.D[2 * CH + l] = __expf(gv);
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt = 0
    }
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };
  // bf16 output rows of a chunk from sO to global memory.
  auto store_o = [&](int ot0, int olen) __attribute__((always_inline)) {
    if constexpr (!F32) {
      const rsrc_t rr = make_rsrc((T*)p.o + ((long)ot0 * p.Hv + h) * VD, (long)olen * p.Hv * VD * (long)sizeof(T));
      const uint32_t rs = (uint32_t)(p.Hv * VD * (int)sizeof(T));
#pragma unroll
      for (int i = threadIdx.x; i < CH * NCH; i += FNT) {
        const int r = i / NCH, c = i % NCH;
        buf_store16<true>(rr, (uint32_t)r * rs + (uint32_t)c * 16u,
                          *reinterpret_cast<const uint4*>(sO + (r * NCH + (c ^ stage_swz<NCH>(r))) * VEC));
      }
    }
  };

  if (cstart < cend) copy_chunk(cstart, ic<0>());
  // The upper tiles (0,1) and (2,3) that the 32-token contraction steps of
  // P Vnew read are always zero: written once here (published by the
  // barrier below), never recomputed.
  if constexpr (MODE == 0 || MODE == 4) {
    for (int i = threadIdx.x; i < PSZ; i += FNT) sP[i] = from_f<T>(0.f);
  }
  wait_copies(cstart, ic<0>());

  // P tiles of this wave (rows of tile ti, columns of tile tj): the ten
  // lower tiles; waves 0-3 take two, waves 4 and 5 one (the two zero tiles
  // in the table's last places belong to no wave).
  const int pcnt = w < 4 ? 2 : (w < 6 ? 1 : 0);
  int pti[2], ptj[2];
  {
    constexpr int TI[12] = {3, 3, 2, 2, 3, 3, 2, 1, 1, 0, 0, 2};
    constexpr int TJ[12] = {0, 1, 0, 1, 2, 3, 2, 0, 1, 0, 1, 3};
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int idx = w < 4 ? 2 * w + m : 8 + (w - 4);
      pti[m] = TI[idx];
      ptj[m] = TJ[idx];
    }
  }
  int prev_t0 = 0, prev_len = 0;
  bool prev_out = false;
  // One chunk from buffer bc, copying chunk jc + 1 into the other buffer;
  // false if the chunk tables are inconsistent (nothing is done then).
  auto step = [&](auto bc, int jc) __attribute__((always_inline)) -> bool {
    constexpr int b = decltype(bc)::value;
    const int t0 = seq0 + jc * CH;
    const int len = min(CH, seq1 - t0);
    if (len <= 0 || t0 < 0 || (long)t0 + len > s.Ttot) return false;
    const bool warm = jc < cbeg || TRANS || st_mode;   // no output for this chunk
    const bool keep = st_mode && jc >= cbeg;             // store the entry state and Vnew
    const bool more = jc + 1 < cend;
    const FusedBufs<T> cur = bufs(bc);
    const T* sW = cur.W;
    const T* sQ = cur.Q;
    const T* sK = cur.K;
    const T* sU = cur.U;
    const float* sG = cur.G;
    const float* sD = cur.D;
    const float* sM = cur.D + CH;
    const float glast = sG[len - 1];
    if (keep && owner) {   // entry state of the chunk, [K][V] rows
      T* hb = (T*)p.hbuf + ((long)h * s.NTtot + c0 + jc) * KD * VD;
      if constexpr (F32) {
#pragma unroll
        for (int rb = 0; rb < NKB; ++rb)
#pragma unroll
          for (int e = 0; e < 4; ++e) hb[(long)(16 * rb + acc_row(e)) * VD + vcol(0)] = hs[rb][0][e];
      } else {
        // A 4x4 transpose within each lane quad gives a lane one K row over
        // the quad's four columns, staged (8 bytes per tile) in the Q
        // buffers, which the states pass does not use; the rows leave as
        // 16-byte pieces after the mid-chunk barrier.
#pragma unroll
        for (int rb = 0; rb < NKB; ++rb) {
          const int r = krow(rb, t & 3);
          *reinterpret_cast<uint2*>((r < CH ? sQ0 : sQ1) + tix(r & (CH - 1), 16 * w + 4 * (t >> 2))) =
              pack4_bf16(quad_t(hs[rb][0]));
        }
      }
    }

    if (!warm && pcnt > 0) {  // P tiles of this wave
      // Masked scaled decays first (they do not depend on the products).
      // The products are formed with swapped operands, so a lane holds row
      // 16i + t over the four columns 16j + 4q + e (one store, no in-quad
      // transpose), whose gate cumsums are one 16-byte read.
      f32x4 dec[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int r = 16 * pti[m] + t, c0 = 16 * ptj[m] + 4 * q;
        const float gr = sG[r];
        const f32x4 gc = *reinterpret_cast<const f32x4*>(sG + c0);
#pragma unroll
        for (int e = 0; e < 4; ++e) dec[m][e] = (r >= c0 + e && r < len) ? p.scale * __expf(gr - gc[e]) : 0.f;
      }
      f32x4 pa[2] = {zero4(), zero4()};
      if constexpr (F32) {
        // Lane quarter q takes the four consecutive K columns 16s + 4q.. of
        // each 16-column slice as one 16-byte read of Q and of K; step e of
        // the slice contracts over column 16s + 4q + e.
#pragma unroll
        for (int k0 = 0; k0 < KD; k0 += 16) {
          f32x4 fa[2], fb[2];
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            fa[m] = *reinterpret_cast<const f32x4*>(sQ + tix(16 * pti[m] + t, k0 + 4 * q));
            fb[m] = *reinterpret_cast<const f32x4*>(sK + tix(16 * ptj[m] + t, k0 + 4 * q));
          }
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int m = 0; m < 2; ++m) pa[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(fb[m][e], fa[m][e], pa[m], 0, 0, 0);
        }
      } else if (pcnt > 1) {
#pragma unroll
        for (int k0 = 0; k0 < KD; k0 += 32) {
          bf16x8 fa[2], fb[2];
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            fa[m] = *reinterpret_cast<const bf16x8*>(sQ + tix(16 * pti[m] + t, k0 + 8 * q));
            fb[m] = *reinterpret_cast<const bf16x8*>(sK + tix(16 * ptj[m] + t, k0 + 8 * q));
          }
#pragma unroll
          for (int m = 0; m < 2; ++m) pa[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[m], fa[m], pa[m], 0, 0, 0);
        }
      } else {   // one tile
#pragma unroll
        for (int k0 = 0; k0 < KD; k0 += 32) {
          const bf16x8 fa = *reinterpret_cast<const bf16x8*>(sQ + tix(16 * pti[0] + t, k0 + 8 * q));
          const bf16x8 fb = *reinterpret_cast<const bf16x8*>(sK + tix(16 * ptj[0] + t, k0 + 8 * q));
          pa[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb, fa, pa[0], 0, 0, 0);
        }
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        if (m < pcnt) {
          const f32x4 pv = dec[m] * pa[m];
          if constexpr (F32) {
            *reinterpret_cast<f32x4*>(sP + (16 * pti[m] + t) * PP + 16 * ptj[m] + 4 * q) = pv;
          } else {
            // row 16i + t, columns 16j + 4q .. +3, which the column
            // permutation keeps adjacent (one 8-byte store)
            const int rr = 16 * pti[m] + t, cc = 16 * ptj[m] + 4 * q;
            const int pc = (cc & ~31) + 8 * ((cc >> 2) & 3) + 4 * ((cc >> 4) & 1);
            *reinterpret_cast<uint2*>(sP + tix8(rr, pc)) = pack4_bf16(pv);
          }
        }
      }
    }

    if (more) {   // the next chunk's tiles, issued once this wave's P reads are out
#pragma unroll
      for (int piece = 0; piece < 4; ++piece) copy_part(jc + 1, ic<1 - b>(), piece);
    }
    f32x4 vn[4][CBW], oa[4][CBW];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int cb = 0; cb < CBW; ++cb) { vn[tt][cb] = zero4(); oa[tt][cb] = zero4(); }
    if (owner) {
      // Vnew = U - W h and Q h.
      if constexpr (F32) {
        // step st of row block rb contracts over K row 16rb + 4q + st, which
        // is where the state accumulator keeps it; the W and Q entries of
        // the four steps are one 16-byte read per token tile
#pragma unroll
        for (int rb = 0; rb < NKB; ++rb) {
          f32x4 aw[4], aq[4];
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            aw[tt] = *reinterpret_cast<const f32x4*>(sW + tix(16 * tt + t, 16 * rb + 4 * q));
            if (!warm) aq[tt] = *reinterpret_cast<const f32x4*>(sQ + tix(16 * tt + t, 16 * rb + 4 * q));
          }
#pragma unroll
          for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
              for (int cb = 0; cb < CBW; ++cb)
                vn[tt][cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(aw[tt][st], hs[rb][cb][st], vn[tt][cb], 0, 0, 0);
              if (!warm) {
#pragma unroll
                for (int cb = 0; cb < CBW; ++cb)
                  oa[tt][cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(aq[tt][st], hs[rb][cb][st], oa[tt][cb], 0, 0, 0);
              }
            }
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < KD / 32; ++ks) {
          bf16x8 aw[4], hb[CBW];
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) aw[tt] = *reinterpret_cast<const bf16x8*>((AP ? sK : sW) + tix(16 * tt + t, 32 * ks + 8 * q));
#pragma unroll
          for (int cb = 0; cb < CBW; ++cb) hb[cb] = pack_b(hs[2 * ks][cb], hs[2 * ks + 1][cb]);
#pragma unroll
          for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int cb = 0; cb < CBW; ++cb) vn[tt][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw[tt], hb[cb], vn[tt][cb], 0, 0, 0);
        }
        if (!warm) {   // Q h after K h: its products fill the K h -> Vnew latency
          // The output products take swapped operands (the A and B fragments
          // have the same register layout), so that oa holds transposed
          // blocks: lane (q, t) has token row 16tt + t over the four value
          // columns 16w + 4q + e, staged as one 8-byte write per tile.
#pragma unroll
          for (int ks = 0; ks < KD / 32; ++ks) {
            bf16x8 aq[4];
            const bf16x8 hb = pack_b(hs[2 * ks][0], hs[2 * ks + 1][0]);
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) aq[tt] = *reinterpret_cast<const bf16x8*>(sQ + tix(16 * tt + t, 32 * ks + 8 * q));
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) oa[tt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hb, aq[tt], oa[tt][0], 0, 0, 0);
          }
        }
      }
      float uv[4][4][CBW];
      if constexpr (!F32 && CBW == 1) {
        // The wave's 16 value columns over a tile's rows 4g..4g+3: one
        // transposing read per tile gives each lane its column's four rows.
        typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
        const int sl = l & 15;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(sU + tix(16 * tt + 4 * q + (sl >> 2), 16 * w + 4 * (sl & 3))));
#pragma unroll
          for (int e = 0; e < 4; ++e) uv[tt][e][0] = no_u ? 0.f : __uint_as_float((uint32_t)(uint16_t)x[e] << 16);
        }
      } else {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int cb = 0; cb < CBW; ++cb)   // (the U tile is not copied for M)
              uv[tt][e][cb] = no_u ? 0.f : to_f(sU[tix(16 * tt + acc_row(e), vcol(cb))]);
      }
      if constexpr (AP) {   // vn holds K h: Vnew = A''(V - Gamma * K h), A'' lower triangular
        const float* sGa = sD + 2 * CH;
        f32x4 xv[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const f32x4 ga = *reinterpret_cast<const f32x4*>(sGa + 16 * tt + 4 * q);
#pragma unroll
          for (int e = 0; e < 4; ++e) xv[tt][e] = uv[tt][e][0] - ga[e] * vn[tt][0][e];
        }
        const bf16x8 xb[2] = {pack_b(xv[0], xv[1]), pack_b(xv[2], xv[3])};
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          vn[tt][0] = zero4();
#pragma unroll
          for (int ks = 0; ks <= tt / 2; ++ks) {
            const uint2 lo = *reinterpret_cast<const uint2*>(sW + tix8(16 * tt + t, 32 * ks + 4 * q));
            const uint2 hi = *reinterpret_cast<const uint2*>(sW + tix8(16 * tt + t, 32 * ks + 16 + 4 * q));
            bf16x8 a;
            __builtin_memcpy(&a, &lo, 8);
            __builtin_memcpy(reinterpret_cast<char*>(&a) + 8, &hi, 8);
            vn[tt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, xb[ks], vn[tt][0], 0, 0, 0);
          }
        }
      }
      f32x4 vd[4][CBW];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const float gmt = sM[16 * tt + t];   // bf16: oa's row is 16tt + t
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * tt + acc_row(e);
          const float d = sD[r];
          const float gm = F32 ? sM[r] : gmt;
#pragma unroll
          for (int cb = 0; cb < CBW; ++cb) {
            if constexpr (!AP) vn[tt][cb][e] = uv[tt][e][cb] - vn[tt][cb][e];
            vd[tt][cb][e] = vn[tt][cb][e] * d;
            oa[tt][cb][e] *= gm;
          }
        }
      }
      if (keep) {   // Vnew token rows
        T* vb = (T*)p.vnew + ((long)h * s.Ttot + t0) * VD;
        if constexpr (F32) {
#pragma unroll
          for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 16 * tt + acc_row(e);
              if (r < len) vb[(long)r * VD + vcol(0)] = vn[tt][0][e];
            }
        } else {   // quad transposes as for the entry state, staged in sO
#pragma unroll
          for (int tt = 0; tt < 4; ++tt)
            *reinterpret_cast<uint2*>(sO + tix(16 * tt + 4 * q + (t & 3), 16 * w + 4 * (t >> 2))) =
                pack4_bf16(quad_t(vn[tt][0]));
        }
      }
      // h' = Gamma_n h + K^T (d * Vnew).
      const float gn = __expf(glast);
#pragma unroll
      for (int rb = 0; rb < NKB; ++rb)
#pragma unroll
        for (int cb = 0; cb < CBW; ++cb) hs[rb][cb] *= gn;
      if constexpr (F32) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int rb = 0; rb < NKB; ++rb) {
              const float ak = sK[tix(16 * tt + 4 * q + st, 16 * rb + t)];
#pragma unroll
              for (int cb = 0; cb < CBW; ++cb)
                hs[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(ak, vd[tt][cb][st], hs[rb][cb], 0, 0, 0);
            }
      } else {
        typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
        const int sl = l & 15;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          bf16x8 ak[NKB], vb[CBW];
#pragma unroll
          for (int rb = 0; rb < NKB; ++rb) {
            const int r0 = 32 * ks + 4 * q + (sl >> 2), cc = 32 * (rb >> 1) + 8 * (sl & 3) + 4 * (rb & 1);
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(sK + tix(r0, cc)));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(sK + tix(r0 + 16, cc)));
            ak[rb] = cat4(lo, hi);
          }
#pragma unroll
          for (int cb = 0; cb < CBW; ++cb) vb[cb] = pack_b(vd[2 * ks][cb], vd[2 * ks + 1][cb]);
#pragma unroll
          for (int rb = 0; rb < NKB; ++rb)
#pragma unroll
            for (int cb = 0; cb < CBW; ++cb) hs[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak[rb], vb[cb], hs[rb][cb], 0, 0, 0);
          if constexpr (SPLITV) {
#pragma unroll
            for (int cb = 0; cb < CBW; ++cb) {
              const bf16x8 vl = pack_b_lo(vd[2 * ks][cb], vd[2 * ks + 1][cb], vb[cb]);
#pragma unroll
              for (int rb = 0; rb < NKB; ++rb) hs[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak[rb], vl, hs[rb][cb], 0, 0, 0);
            }
          }
        }
      }
    }
    if (prev_out) store_o(prev_t0, prev_len);
    // P complete; the previous chunk's output rows are out of LDS; the staged
    // entry state is in.  A warm step that stores no state writes none of
    // these (its copies go to the other buffer, which the end-of-step barrier
    // publishes), so it skips this barrier: the output pass's warmup and
    // every transition step.
    if (!warm || keep) lds_barrier();
    if (!F32 && keep) {   // the staged entry state and Vnew rows, 16-byte pieces
      // (non-temporal: the gradient kernel reads them only after the reverse pass)
      typedef unsigned u32x4nt __attribute__((ext_vector_type(4)));
      T* hb = (T*)p.hbuf + ((long)h * s.NTtot + c0 + jc) * KD * VD;
#pragma unroll
      for (int i = threadIdx.x; i < KD * NCH; i += FNT) {
        const int r = i / NCH, c = i % NCH;
        const T* src = (r < CH ? sQ0 : sQ1) + ((r & (CH - 1)) * NCH + (c ^ stage_swz<NCH>(r))) * VEC;
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4nt*>(src), reinterpret_cast<u32x4nt*>(hb + (long)r * VD + c * VEC));
      }
      const rsrc_t vr = make_rsrc((T*)p.vnew + ((long)h * s.Ttot + t0) * VD, (long)len * VD * (long)sizeof(T));
#pragma unroll
      for (int i = threadIdx.x; i < CH * NCH; i += FNT) {
        const int r = i / NCH, c = i % NCH;
        buf_store16<true>(vr, (uint32_t)(r * VD + c * VEC) * (uint32_t)sizeof(T),
                          *reinterpret_cast<const uint4*>(sO + (r * NCH + (c ^ stage_swz<NCH>(r))) * VEC));
      }
    }

    if (!warm && owner) {  // O += P Vnew
      if constexpr (F32) {
        // step st of token tile tp contracts over token 16tp + 4q + st, as
        // Vnew's accumulator holds it; P's four entries are one 16-byte read
#pragma unroll
        for (int tp = 0; tp < 4; ++tp) {
          f32x4 ap[4];
#pragma unroll
          for (int tt = tp; tt < 4; ++tt) ap[tt] = *reinterpret_cast<const f32x4*>(sP + (16 * tt + t) * PP + 16 * tp + 4 * q);
#pragma unroll
          for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int tt = tp; tt < 4; ++tt)
#pragma unroll
              for (int cb = 0; cb < CBW; ++cb)
                oa[tt][cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(ap[tt][st], vn[tp][cb][st], oa[tt][cb], 0, 0, 0);
        }
        // fp32 output straight from the accumulators (16 lanes cover 64 contiguous bytes)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 16 * tt + acc_row(e);
            if (r < len) {
#pragma unroll
              for (int cb = 0; cb < CBW; ++cb) ((T*)p.o)[((long)(t0 + r) * p.Hv + h) * VD + vcol(cb)] = oa[tt][cb][e];
            }
          }
      } else {
        bf16x8 ap[2][4];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int tt = 2 * ks; tt < 4; ++tt) ap[ks][tt] = *reinterpret_cast<const bf16x8*>(sP + tix8(16 * tt + t, 32 * ks + 8 * q));
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          bf16x8 vb[CBW];
#pragma unroll
          for (int cb = 0; cb < CBW; ++cb) vb[cb] = pack_b(vn[2 * ks][cb], vn[2 * ks + 1][cb]);
#pragma unroll
          for (int tt = 2 * ks; tt < 4; ++tt)
#pragma unroll
            for (int cb = 0; cb < CBW; ++cb) oa[tt][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb[cb], ap[ks][tt], oa[tt][cb], 0, 0, 0);
          if constexpr (SPLITV) {
#pragma unroll
            for (int cb = 0; cb < CBW; ++cb) {
              const bf16x8 vl = pack_b_lo(vn[2 * ks][cb], vn[2 * ks + 1][cb], vb[cb]);
#pragma unroll
              for (int tt = 2 * ks; tt < 4; ++tt) oa[tt][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vl, ap[ks][tt], oa[tt][cb], 0, 0, 0);
            }
          }
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)   // row 16tt + t, columns 16w + 4q .. +3
          *reinterpret_cast<uint2*>(sO + tix(16 * tt + t, 16 * w + 4 * q)) = pack4_bf16(oa[tt][0]);
      }
    }
    wait_copies(jc + 1, ic<1 - b>());   // the next chunk's tiles have landed; the output rows are staged
    prev_out = !warm && !F32;
    prev_t0 = t0;
    prev_len = len;
    return true;
  };
  for (int jc = cstart; jc < cend; jc += 2) {
    if (!step(ic<0>(), jc) || jc + 1 >= cend || !step(ic<1>(), jc + 1)) break;
  }
  if (prev_out) store_o(prev_t0, prev_len);

  if (TRANS && owner) {
    float* dst = p.segtr + (((long)h * p.total_segs + gseg) * 2 + part) * KD * VD;
#pragma unroll
    for (int rb = 0; rb < NKB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CBW; ++cb)
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[(long)(F32 ? 16 * rb + acc_row(e) : krow(rb, e)) * VD + vcol(cb)] = hs[rb][cb][e];
  }
  if (write_final && p.ht && owner) {
#pragma unroll
    for (int rb = 0; rb < NKB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CBW; ++cb)
#pragma unroll
        for (int e = 0; e < 4; ++e) p.ht[hbase + (long)(F32 ? 16 * rb + acc_row(e) : krow(rb, e)) * VD + vcol(cb)] = hs[rb][cb][e];
  }
}

// -------------------------------------------------------------- k_segscan --
// Exact start states of the CP segments of heads that fail the warmup
// certificate: h_1 = b_0 (the first segment's end state from the initial
// state), h_{s+1} = M_s h_s + b_s.  Reverse mode (backward): the state
// gradient entering segment s from its end is g_s = M_{s+1}^T g_{s+1} + d_{s+1},
// g_{nseg-2} = d_{nseg-1} (the last segment run from the final-state gradient),
// where d_s is the reverse pass over segment s from a zero gradient.  State columns are independent, so one
// workgroup per (sequence, value head, 16-column block) with KD/16 waves;
// wave w produces rows 16w..16w+15.  The A operand (rows of M_s) comes
// straight from memory into registers, one step ahead; the state slice
// lives in LDS transposed (column-major), double-buffered, so each lane's B
// operand is one 16-byte read and each step needs one barrier.
template <int KD>
__global__ __launch_bounds__(KD * 4) void k_segscan(ScanParams p, int total_items) {
  constexpr int VD = KD, NKB = KD / 16, NCB = VD / 16, PH = KD + 4;
  __shared__ __align__(16) float sH[2][16 * PH];
  const SeqTables& s = p.s;
  const int u = xcd_remap(blockIdx.x, total_items);
  if (u >= total_items) return;
  const int cb = u % NCB, h = (u / NCB) % p.Hv, n = u / (NCB * p.Hv);
  if (n >= s.N) return;
  const int nseg = s.seg_at(n + 1) - s.seg_at(n);
  const int c0 = s.chunk_at(n);
  const int L = p.seg_chunks;
  if (nseg <= 1 || c0 < 0) return;
  const int nch = s.chunk_at(n + 1) - c0;
  if (p.hflag ? p.hflag[(long)n * p.Hv + h] != 0
              : head_certified(p.cert + (long)h * s.NTtot + c0, nseg, nch, L, p.warmup, p.log_eps, p.rev_cert != 0))
    return;   // certified: the warmup path needs no start states
  const int w = wave_id(), l = lane_id(), q = l >> 4, t = l & 15;
  const int col = 16 * cb + t, row0 = 16 * w + 4 * q;
  const long head = (long)h * p.total_segs + s.seg_at(n);
  auto tr = [&](int sg, int part) { return p.segtr + ((head + sg) * 2 + part) * KD * VD; };
  auto load_m = [&](int sg, f32x4 (&a)[NKB]) {
    if (p.rev) {   // M^T: lane reads column 16w + t of M, rows 16rb + 4q .. +3
      const float* M = tr(sg, 0) + (long)(4 * q) * KD + 16 * w + t;
#pragma unroll
      for (int rb = 0; rb < NKB; ++rb)
#pragma unroll
        for (int e = 0; e < 4; ++e) a[rb][e] = M[(long)(16 * rb + e) * KD];
    } else {
      const float* M = tr(sg, 0) + (long)(16 * w + t) * KD + 4 * q;
#pragma unroll
      for (int rb = 0; rb < NKB; ++rb) a[rb] = *reinterpret_cast<const f32x4*>(M + 16 * rb);
    }
  };
  auto load_b = [&](int sg, f32x4& b) {
    const float* B = tr(sg, 1) + (long)row0 * VD + col;
#pragma unroll
    for (int e = 0; e < 4; ++e) b[e] = B[(long)e * VD];
  };
  // Step i stores slot sx(i) and then applies transition sx(i): forward
  // slots 1 .. nseg-1 from b_0; reverse slots nseg-2 .. 0 from d_{nseg-1}.
  auto sx = [&](int i) { return p.rev ? nseg - 1 - i : i; };
  f32x4 hs, bn, a[NKB];
  load_b(p.rev ? nseg - 1 : 0, hs);
  if (nseg > 2) { load_m(sx(1), a); load_b(sx(1), bn); }
  for (int sg = 1; sg < nseg; ++sg) {
    float* dst = p.hstart + (head + sx(sg)) * KD * VD + (long)row0 * VD + col;
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[(long)e * VD] = hs[e];
    if (sg == nseg - 1) break;
    float* buf = sH[sg & 1];
    *reinterpret_cast<f32x4*>(buf + t * PH + row0) = hs;
    __syncthreads();
    f32x4 an[NKB], bnn = bn;
    const bool more = sg + 1 < nseg - 1;
    if (more) { load_m(sx(sg + 1), an); load_b(sx(sg + 1), bnn); }
    f32x4 acc0 = bn, acc1 = zero4();
#pragma unroll
    for (int rb = 0; rb < NKB; rb += 2) {
      acc0 = mm(acc0, a[rb], *reinterpret_cast<const f32x4*>(buf + t * PH + 16 * rb + 4 * q));
      if (rb + 1 < NKB) acc1 = mm(acc1, a[rb + 1], *reinterpret_cast<const f32x4*>(buf + t * PH + 16 * (rb + 1) + 4 * q));
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) hs[e] = acc0[e] + acc1[e];
    if (more) {
#pragma unroll
      for (int rb = 0; rb < NKB; ++rb) a[rb] = an[rb];
      bn = bnn;
    }
  }
}

// ------------------------------------------------------------- launchers --
#define GDR_LAUNCH(name, kern, grid, st, ...)        \
  do {                                               \
    timing_before(name, st);                         \
    hipLaunchKernelGGL(kern, grid, dim3(NTHR), 0, st, __VA_ARGS__); \
    err = hipGetLastError();                         \
    timing_after(st);                                \
  } while (0)

hipError_t launch_plan(const PlanParams& p, hipStream_t st) {
  timing_before("plan", st);
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(1024), 0, st, p);
  hipError_t err = hipGetLastError();
  timing_after(st);
  return err;
}

static unsigned padded_grid(long total) { return (unsigned)(((total + 7) / 8) * 8); }

template <typename T, int KD>
static hipError_t intra_impl(const IntraParams& p, hipStream_t st) {
  hipError_t err;
  // bf16: A diag(beta) rows, one item per wave; fp32: W and U, a persistent
  // grid of three workgroups per CU, each over a contiguous item range
  constexpr bool BF = std::is_same<T, bf16>::value;
  if (BF ? p.Au == nullptr : (p.W == nullptr || p.U == nullptr)) return hipErrorInvalidValue;
  const long total = (long)p.s.NTtot * p.Hv;
  if constexpr (BF) {
    const int nw = (int)((total + NWAVE - 1) / NWAVE);
    if (p.A_bf && (p.A_ws || p.A_out)) return hipErrorInvalidValue;   // one form of A per call
    if (p.A_bf) {
      GDR_LAUNCH("intra_wy", (k_intra_w<KD, 2>), dim3(padded_grid(nw)), st, p, (int)total, nw);
    } else if (p.A_ws || p.A_out) {
      GDR_LAUNCH("intra_wy", (k_intra_w<KD, 1>), dim3(padded_grid(nw)), st, p, (int)total, nw);
    } else {
      GDR_LAUNCH("intra_wy", (k_intra_w<KD, 0>), dim3(padded_grid(nw)), st, p, (int)total, nw);
    }
  } else {
    const int nwg = (int)std::min<long>(padded_grid(total), 3 * 256);
    const int per_wg = (int)((total + nwg - 1) / nwg);
    GDR_LAUNCH("intra_wy", (k_intra<T, KD>), dim3(nwg), st, p, (int)total, per_wg, nwg);
  }
  return err;
}

template <typename T, int KD, int BV>
static hipError_t state_impl(const StateParams& p, int total_segs, bool rows, hipStream_t st) {
  hipError_t err;
  const int total = total_segs * p.Hv * p.nvb;
  if (!rows) return hipErrorInvalidValue;
  GDR_LAUNCH("chunk_state_rows", (k_state<T, KD, BV, true>), dim3(padded_grid(total)), st, p, total);
  return err;
}

template <typename T, int KD>
static hipError_t fused_impl(const FusedParams& p, int total_segs, hipStream_t st) {
  const int total = total_segs * p.Hv * (p.trans ? 2 : 1);
  const bool states = p.hbuf != nullptr && !p.trans;
  // bf16 passes read A diag(beta) and V; fp32 passes read W and U
  constexpr bool F32 = std::is_same<T, float>::value;
  const bool apath = !F32;
  // (with no token at all the pass only writes the final states: nothing is read)
  if (p.s.Ttot > 0 && (apath ? (p.Au == nullptr || p.v == nullptr) : (p.W == nullptr || p.U == nullptr)))
    return hipErrorInvalidValue;
  // with a segment order: 8 XCDs x G slots per round of head groups
  const unsigned grid = (!p.trans && p.s.seg_order)
      ? (unsigned)(8 * (p.Hv / p.Hq) * (((long)total_segs * p.Hq + 7) / 8)) : padded_grid(total);
  if (!p.trans && p.s.seg_order && total_segs > 1024) return hipErrorInvalidValue;
  timing_before(p.trans ? "cp_transition" : states ? "chunk_states" : "chunk_fused", st);
  if (p.trans && apath) hipLaunchKernelGGL((k_fused<T, KD, 2>), dim3(grid), dim3(FNT), 0, st, p, total);
  else if (p.trans) hipLaunchKernelGGL((k_fused<T, KD, 3>), dim3(grid), dim3(FNT), 0, st, p, total);
  else if (states) hipLaunchKernelGGL((k_fused<T, KD, 1>), dim3(grid), dim3(FNT), 0, st, p, total);
  else if constexpr (!F32) {
    if (p.split_vnew) hipLaunchKernelGGL((k_fused<T, KD, 4>), dim3(grid), dim3(FNT), 0, st, p, total);
    else hipLaunchKernelGGL((k_fused<T, KD, 0>), dim3(grid), dim3(FNT), 0, st, p, total);
  } else {
    hipLaunchKernelGGL((k_fused<T, KD, 0>), dim3(grid), dim3(FNT), 0, st, p, total);
  }
  hipError_t err = hipGetLastError();
  timing_after(st);
  return err;
}

hipError_t launch_segscan(int KD, const ScanParams& p, int total_items, hipStream_t st) {
  timing_before("cp_scan", st);
  total_items *= KD / 16;   // one workgroup per 16-column block
  const dim3 grid(padded_grid(total_items)), block(KD * 4);
  if (KD == 32) hipLaunchKernelGGL(k_segscan<32>, grid, block, 0, st, p, total_items);
  else if (KD == 64) hipLaunchKernelGGL(k_segscan<64>, grid, block, 0, st, p, total_items);
  else hipLaunchKernelGGL(k_segscan<128>, grid, block, 0, st, p, total_items);
  hipError_t err = hipGetLastError();
  timing_after(st);
  return err;
}

hipError_t launch_intra(DType dt, int KD, const IntraParams& p, hipStream_t st) {
  if (dt == DType::BF16) {
    if (KD == 32) return intra_impl<bf16, 32>(p, st);
    if (KD == 64) return intra_impl<bf16, 64>(p, st);
    if (KD == 128) return intra_impl<bf16, 128>(p, st);
  } else {
    if (KD == 32) return intra_impl<float, 32>(p, st);
    if (KD == 64) return intra_impl<float, 64>(p, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_state(DType dt, int KD, int BV, const StateParams& p, int total_segs, bool rows,
                        hipStream_t st) {
  if (dt == DType::BF16) {
    if (KD == 32 && BV == 32) return state_impl<bf16, 32, 32>(p, total_segs, rows, st);
    if (KD == 64 && BV == 32) return state_impl<bf16, 64, 32>(p, total_segs, rows, st);
    if (KD == 128 && BV == 64) return state_impl<bf16, 128, 64>(p, total_segs, rows, st);
  } else {
    if (KD == 32 && BV == 32) return state_impl<float, 32, 32>(p, total_segs, rows, st);
    if (KD == 64 && BV == 32) return state_impl<float, 64, 32>(p, total_segs, rows, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fused(DType dt, int KD, const FusedParams& p, int total_segs, hipStream_t st) {
  if (dt == DType::BF16) {
    if (KD == 32) return fused_impl<bf16, 32>(p, total_segs, st);
    if (KD == 64) return fused_impl<bf16, 64>(p, total_segs, st);
    if (KD == 128) return fused_impl<bf16, 128>(p, total_segs, st);
  } else {
    if (KD == 32) return fused_impl<float, 32>(p, total_segs, st);
    if (KD == 64) return fused_impl<float, 64>(p, total_segs, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdr
