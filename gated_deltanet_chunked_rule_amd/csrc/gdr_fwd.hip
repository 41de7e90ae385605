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
//   k_intra   per (chunk, value head): gate cumsum, K K^T, blocked fp32
//             triangular inverse, W and U on MFMA            [fully parallel]
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
}

// Locates chunk c: sequence n, first token t0 and valid length; false if the
// device tables disagree with the grid (then the workgroup writes nothing).
__device__ __forceinline__ bool locate_chunk(const SeqTables& s, int c, int& n, int& t0, int& len) {
  if (c >= s.NTtot) return false;
  n = find_seq(s.chunk_off, s.N, c);
  t0 = s.cu[n] + (c - s.chunk_off[n]) * CH;
  len = min(CH, s.cu[n + 1] - t0);
  return len > 0 && t0 >= 0 && (long)t0 + len <= s.Ttot;
}

// --------------------------------------------------------------- k_intra --
// Persistent: each workgroup walks a contiguous range of (chunk, value head)
// items (value heads of one chunk adjacent, so the shared K tile is an L2
// hit) and loads the next item's K, V, g and beta into a second register set
// while the current one is computed.  Wave i owns row block i (tokens
// 16i..16i+15) of A, W and U.  Per item:
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

// acc + X Y for 16 x 16 fp32 tiles in LDS (pitch P); contraction index 4s + q
// at step s for lane group q.
template <int P>
__device__ __forceinline__ f32x4 mm_ll(f32x4 acc, const float* X, const float* Y) {
  const int l = lane_id(), q = l >> 4, t = l & 15;
#pragma unroll
  for (int s = 0; s < 4; ++s)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(X[t * P + 4 * s + q], Y[(4 * s + q) * P + t], acc, 0, 0, 0);
  return acc;
}
// acc + X R, R a 16 x 16 accumulator tile in registers (lane group q holds
// its rows 4q..4q+3): at step s group q contracts over index 4q + s, for
// which it holds R's row in element s.
template <int P>
__device__ __forceinline__ f32x4 mm_lr(f32x4 acc, const float* X, f32x4 R) {
  const int l = lane_id(), q = l >> 4, t = l & 15;
#pragma unroll
  for (int s = 0; s < 4; ++s)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(X[t * P + 4 * q + s], R[s], acc, 0, 0, 0);
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

// Lower tiles (i, j) of K K^T computed by wave w (n-th of kk_count(w)).
__device__ __forceinline__ int kk_count(int w) { return (w & 1) ? 2 : 3; }
__device__ __forceinline__ void kk_tile(int w, int n, int& i, int& j) {
  // w0: (0,0) (3,0) (3,1)   w1: (1,0) (1,1)   w2: (2,0) (2,1) (2,2)   w3: (3,2) (3,3)
  if (w == 0) { i = n == 0 ? 0 : 3; j = n == 0 ? 0 : n - 1; }
  else if (w == 1) { i = 1; j = n; }
  else if (w == 2) { i = 2; j = n; }
  else { i = 3; j = 2 + n; }
}

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
  __shared__ __align__(16) char smem[2 * SZ_K + SZ_F + SZ_X];
  __shared__ float sG[CH], sB[CH];
  __shared__ int sFlag[NWAVE];
  T* sK = reinterpret_cast<T*>(smem);
  T* sV = reinterpret_cast<T*>(smem + SZ_K);
  float* sF = reinterpret_cast<float*>(smem + 2 * SZ_K);
  T* sAw = reinterpret_cast<T*>(smem + 2 * SZ_K + (F32 ? SZ_F : 0));  // A'^T  [token j][token i]
  T* sAu = sAw + CH * PA;                                              // A''^T

  const SeqTables& s = p.s;
  const int x = xcd_remap(blockIdx.x, nwg);
  const int u0 = x * per_wg, u1 = min(total_items, u0 + per_wg);
  if (u0 >= u1) return;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  const int q = l >> 4, t = l & 15;
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
      const int cnt = kk_count(w);
      f32x4 acc[3];
      int ti[3], tj[3];
#pragma unroll
      for (int n = 0; n < 3; ++n) {
        acc[n] = zero4();
        kk_tile(w, n, ti[n], tj[n]);
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
      const int any_bad = sFlag[0] | sFlag[1] | sFlag[2] | sFlag[3];
      p.cert[(long)h * s.NTtot + it.c] = any_bad ? INFINITY : sG[len - 1];
    }

    // 3. Row block w of A into registers a0..a3 (tile j), zero above the diagonal.
    f32x4 a0 = zero4(), a1 = zero4(), a2 = zero4(), a3 = zero4();
    if (p.A_in) {
      const float* src = p.A_in + ((long)t0 * p.Hv + h) * CH;
      const long rs = (long)p.Hv * CH;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * w + acc_row(e);
        if (r < len) {
          const float* row = src + (long)r * rs;
          if (0 <= w && t < len) a0[e] = row[t];
          if (1 <= w && 16 + t < len) a1[e] = row[16 + t];
          if (2 <= w && 32 + t < len) a2[e] = row[32 + t];
          if (3 <= w && 48 + t < len) a3[e] = row[48 + t];
        }
      }
    } else {
      // Diagonal block by forward substitution (lane l < 16 solves column l),
      // written over L_ww.
      if (l < 16) {
        float xs[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float acc = (r == l) ? 1.f : 0.f;
          const float* Lr = sF + (16 * w + r) * PF + 16 * w;
#pragma unroll
          for (int jj = 0; jj < r; ++jj) acc -= Lr[jj] * xs[jj];
          xs[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sF[(16 * w + r) * PF + 16 * w + l] = xs[r];
      }
      wave_sync();
      // M_wj = A_ww L_wj over L_wj.
      for (int j = 0; j < w; ++j) st_acc<PF>(tile(w, j), mm_ll<PF>(zero4(), tile(w, w), tile(w, j)));
      lds_barrier();
      const f32x4 dg = ld_acc<PF>(tile(w, w));
      if (w == 0) {
        a0 = dg;
      } else if (w == 1) {
        a0 = -mm_ll<PF>(zero4(), tile(1, 0), tile(0, 0));
        a1 = dg;
      } else if (w == 2) {
        const f32x4 t10 = mm_ll<PF>(zero4(), tile(1, 0), tile(0, 0));
        a0 = mm_lr<PF>(-mm_ll<PF>(zero4(), tile(2, 0), tile(0, 0)), tile(2, 1), t10);
        a1 = -mm_ll<PF>(zero4(), tile(2, 1), tile(1, 1));
        a2 = dg;
      } else {
        const f32x4 t10 = mm_ll<PF>(zero4(), tile(1, 0), tile(0, 0));
        const f32x4 t21 = mm_ll<PF>(zero4(), tile(2, 1), tile(1, 1));
        const f32x4 a20 = mm_lr<PF>(-mm_ll<PF>(zero4(), tile(2, 0), tile(0, 0)), tile(2, 1), t10);
        a0 = mm_lr<PF>(mm_lr<PF>(-mm_ll<PF>(zero4(), tile(3, 0), tile(0, 0)), tile(3, 1), t10), tile(3, 2), -a20);
        a1 = mm_lr<PF>(-mm_ll<PF>(zero4(), tile(3, 1), tile(1, 1)), tile(3, 2), t21);
        a2 = -mm_ll<PF>(zero4(), tile(3, 2), tile(2, 2));
        a3 = dg;
      }
    }
    if (p.A_ws || p.A_out) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * w + acc_row(e);
        if (r < len) {
          const float v4[4] = {a0[e], a1[e], a2[e], a3[e]};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (p.A_ws) p.A_ws[((long)h * s.Ttot + t0 + r) * CH + 16 * j + t] = v4[j];
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
    const int nks = F32 ? 4 * (w + 1) : (w + 2) / 2;  // contraction steps (A' is zero beyond 16(w+1))
    const int ntile = F32 ? w + 1 : 2 * nks;          // A' tiles the steps read
    {
      const f32x4 av[4] = {a0, a1, a2, a3};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j < ntile) {
          acc_store_t<T, PA>(sAw, 16 * w, 16 * j, av[j], sw[j]);
          acc_store_t<T, PA>(sAu, 16 * w, 16 * j, av[j], su[j]);
        }
      }
    }
    wave_sync();

    // 5. W = A' K, U = A'' V for row block w.
    auto gemm_store = [&](const T* sAT, const T* sX, void* dst, int D) {
      f32x4 acc[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[j] = zero4();
      for (int ks = 0; ks < nks; ++ks) {
        if constexpr (F32) {
          const float a = sAT[(4 * ks + q) * PA + 16 * w + t];
#pragma unroll
          for (int j = 0; j < NT; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, sX[(4 * ks + q) * PK + 16 * j + t], acc[j], 0, 0, 0);
        } else {
          const bf16x8 a = tr_frag(sAT + 32 * ks * PA + 16 * w, PA);
#pragma unroll
          for (int j = 0; j < NT; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, tr_frag(sX + 32 * ks * PK + 16 * j, PK), acc[j], 0, 0, 0);
        }
      }
      const rsrc_t rr = make_rsrc((const T*)dst + ((long)h * s.Ttot + t0) * D, (long)len * D * (long)sizeof(T));
#pragma unroll
      for (int e = 0; e < 4; ++e)
        store_acc_row<T, NT>(rr, (uint32_t)(((16 * w + acc_row(e)) * D + NT * t) * (int)sizeof(T)), acc, e);
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
  const int n = find_seq(s.seg_off, s.N, item);
  const int pseg = item - s.seg_off[n];
  const int nseg = s.seg_off[n + 1] - s.seg_off[n];
  const int c0 = s.chunk_off[n];
  const int nch = s.chunk_off[n + 1] - c0;
  if (pseg < 0 || pseg >= nseg || c0 < 0 || c0 + nch > s.NTtot) return;
  const int L = p.seg_chunks;
  const int hk = h / (p.Hv / p.Hq);
  const int w = wave_id();

  // A head is certified when every warmup window's gate mass is small enough
  // (all segments of the head evaluate the same test, so they agree).
  int ok = 1;
  for (int q = 1 + (int)threadIdx.x; q < nseg; q += NTHR) {
    const int ws = q * L - p.warmup;
    if (ws > 0) {
      float sum = 0.f;
      for (int cc = ws; cc < q * L; ++cc) sum += p.cert[(long)h * s.NTtot + c0 + cc];
      if (!(sum <= p.log_eps)) ok = 0;
    }
  }
  const bool certified = !__syncthreads_or(!ok);
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
    const int t0 = s.cu[n] + min(jc, cend - 1) * CH;
    const int len = valid ? min(CH, s.cu[n + 1] - t0) : 0;
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
    const int t0 = s.cu[n] + jc * CH;
    const int len = min(CH, s.cu[n + 1] - t0);
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
// value head, CP segment) covering all V columns, so W, K, Q and P are staged
// once per chunk and the chunk states never leave the chip.  Per chunk:
//   P^T = lower(D * K Q^T) * s      (from K and Q rows; skipped in warmup)
//   Vnew = U - W h,  O = s Gamma (Q h) + P Vnew   (W h and Q h share B tiles)
//   h' = Gamma_n h + (diag(e^{gamma_n - gamma}) K)^T Vnew
// Waves: output tiles (rows 16*(w%4), column half w/4); state tiles 8 per wave.
template <typename T, int KD>
__global__ __launch_bounds__(512) void k_fused(FusedParams p, int total_items) {
  constexpr int NT = 512, NW = 8;
  constexpr int VD = KD;
  constexpr int PK = Pitch<T, KD>::value;
  constexpr int PT = Pitch<T, CH>::value;
  constexpr int NKB = KD / 16, NVB = VD / 16;
  constexpr int NST = NKB * NVB;
  constexpr int HT = (NST + NW - 1) / NW;
  constexpr int OCB = NVB / 2;
  static_assert(NVB % 2 == 0, "V must split into two column halves");
  __shared__ __align__(16) T sW[CH * PK];     // W rows; O staging after W h
  __shared__ __align__(16) T sQ[CH * PK];
  __shared__ __align__(16) T sK[CH * PK];
  __shared__ __align__(16) T sU[CH * PK];
  __shared__ __align__(16) T sKdT[KD * PT];   // e^{gamma_n - gamma_t} k_t[d] as [d][t]
  __shared__ __align__(16) T shT[VD * PK];    // h[d][v] as [v][d]
  __shared__ __align__(16) T sVt[VD * PT];    // Vnew[t][v] as [v][t]
  __shared__ __align__(16) T sP[CH * PT];     // s P[t][s] rows
  __shared__ float sG[CH];

  const SeqTables& s = p.s;
  const int u = xcd_remap(blockIdx.x, total_items);
  if (u >= total_items) return;
  const int h = u % p.Hv;
  const int item = u / p.Hv;
  const int n = find_seq(s.seg_off, s.N, item);
  const int pseg = item - s.seg_off[n];
  const int nseg = s.seg_off[n + 1] - s.seg_off[n];
  const int c0 = s.chunk_off[n];
  const int nch = s.chunk_off[n + 1] - c0;
  if (pseg < 0 || pseg >= nseg || c0 < 0 || c0 + nch > s.NTtot) return;
  const int L = p.seg_chunks;
  const int hk = h / (p.Hv / p.Hq);
  const int w = wave_id(), l = lane_id();
  const int orb = w & 3, ocol = (w >> 2) * OCB;   // output row block, first column tile

  int ok = 1;
  for (int q = 1 + (int)threadIdx.x; q < nseg; q += NT) {
    const int ws = q * L - p.warmup;
    if (ws > 0) {
      float sum = 0.f;
      for (int cc = ws; cc < q * L; ++cc) sum += p.cert[(long)h * s.NTtot + c0 + cc];
      if (!(sum <= p.log_eps)) ok = 0;
    }
  }
  const bool certified = !__syncthreads_or(!ok);
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

  f32x4 hacc[HT];
#pragma unroll
  for (int i = 0; i < HT; ++i) {
    const int ti = w * HT + i, rb = ti / NVB, cb = ti % NVB;
    hacc[i] = zero4();
    if (ti < NST && cstart == 0 && p.h0) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        hacc[i][e] = p.h0[(((long)n * p.Hv + h) * KD + 16 * rb + acc_row(e)) * VD + 16 * cb + acc_col()];
    }
  }

  TileRegs<T, CH, KD, NT> rw, ru;
  TileCols<T, KD, NW> rq, rk;
  float gam_next = 0.f, glast_next = 0.f;
  // Loads of chunk jc into registers.  Issued unconditionally (a chunk past
  // the segment gets an empty range: zeros, no memory traffic) so that no
  // control-flow join forces the compiler to wait for them early.
  auto prefetch = [&](int jc) {
    const bool valid = jc < cend;
    const int t0 = s.cu[n] + min(jc, cend - 1) * CH;
    const int len = valid ? min(CH, s.cu[n + 1] - t0) : 0;
    const int lenq = (jc >= cbeg) ? len : 0;
    rw.load((const T*)p.W + ((long)h * s.Ttot + t0) * KD, KD, len);
    ru.load((const T*)p.U + ((long)h * s.Ttot + t0) * VD, VD, len);
    rk.load((const T*)p.k + ((long)t0 * p.Hq + hk) * KD, (long)p.Hq * KD, len);
    rq.load((const T*)p.q + ((long)t0 * p.Hq + hk) * KD, (long)p.Hq * KD, lenq);
    const rsrc_t gr = make_rsrc(p.gcum + (long)h * s.Ttot + t0, (long)len * 4);
    glast_next = buf_load_f32(gr, (uint32_t)(len - 1) * 4u);
    const float gv = buf_load_f32(gr, (uint32_t)l * 4u);
    gam_next = (l < len) ? gv : glast_next;
  };
  if (cstart < cend) prefetch(cstart);

  for (int jc = cstart; jc < cend; ++jc) {
    const int t0 = s.cu[n] + jc * CH;
    const int len = min(CH, s.cu[n + 1] - t0);
    if (len <= 0 || t0 < 0 || (long)t0 + len > s.Ttot) break;
    const bool warm = jc < cbeg;
    const float glast = glast_next, gam = gam_next;
    rw.template store<PK>(sW);
    ru.template store<PK>(sU);
    rk.template store_t<PT>(sKdT, (l < len) ? __expf(glast - gam) : 0.f);
    if (!warm) {
      rk.template store<PK>(sK);
      rq.template store<PK>(sQ);
    }
    if (w == 0) sG[l] = gam;
#pragma unroll
    for (int i = 0; i < HT; ++i) {
      const int ti = w * HT + i;
      if (ti < NST) acc_store_t<T, PK>(shT, 16 * (ti / NVB), 16 * (ti % NVB), hacc[i]);
    }
    lds_barrier();
    prefetch(jc + 1);

    if (!warm) {  // s P as rows [t][s], from P^T tiles (s-block w%4, t-blocks of this half)
      const int is = w & 3, jt0 = 2 * (w >> 2);
      f32x4 a2[2] = {zero4(), zero4()};
      mma_row<T, KD, 2, PK, 1, 1, PK>(a2, sK + 16 * is * PK, sQ + 16 * jt0 * PK);
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int jt = jt0 + jj;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int sidx = 16 * is + acc_row(e), t = 16 * jt + acc_col();
          a2[jj][e] = (t >= sidx) ? p.scale * __expf(sG[t] - sG[sidx]) * a2[jj][e] : 0.f;
        }
        acc_store_t<T, PT>(sP, 16 * is, 16 * jt, a2[jj]);
      }
    }
    f32x4 oacc[OCB];
    {  // Vnew = U - W h and (if not warm) Q h, sharing the h^T operand tiles
      f32x4 vacc[OCB];
#pragma unroll
      for (int j = 0; j < OCB; ++j) { vacc[j] = zero4(); oacc[j] = zero4(); }
      constexpr int KS = Mma<T>::KSTEP;
      if (!warm) {
#pragma unroll
        for (int k0 = 0; k0 < KD; k0 += KS) {
          const auto fw = Mma<T>::template load<PK, 1>(sW + 16 * orb * PK + k0);
          const auto fq = Mma<T>::template load<PK, 1>(sQ + 16 * orb * PK + k0);
#pragma unroll
          for (int j = 0; j < OCB; ++j) {
            const auto fb = Mma<T>::template load<PK, 1>(shT + 16 * (ocol + j) * PK + k0);
            vacc[j] = Mma<T>::op(fw, fb, vacc[j]);
            oacc[j] = Mma<T>::op(fq, fb, oacc[j]);
          }
        }
      } else {
        mma_row<T, KD, OCB, PK, 1, 1, PK>(vacc, sW + 16 * orb * PK, shT + 16 * ocol * PK);
      }
#pragma unroll
      for (int j = 0; j < OCB; ++j) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          vacc[j][e] = to_f(sU[(16 * orb + acc_row(e)) * PK + 16 * (ocol + j) + acc_col()]) - vacc[j][e];
        acc_store_t<T, PT>(sVt, 16 * orb, 16 * (ocol + j), vacc[j]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float gm = p.scale * __expf(sG[16 * orb + acc_row(e)]);
#pragma unroll
        for (int j = 0; j < OCB; ++j) oacc[j][e] *= gm;
      }
    }
    lds_barrier();

    if (!warm) {  // O += s P Vnew, staged as rows in sW
      mma_row<T, CH, OCB, PT, 1, 1, PT>(oacc, sP + 16 * orb * PT, sVt + 16 * ocol * PT, 16 * (orb + 1));
#pragma unroll
      for (int j = 0; j < OCB; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sW[(16 * orb + acc_row(e)) * PK + 16 * (ocol + j) + acc_col()] = from_f<T>(oacc[j][e]);
    }
    const float dlast = __expf(glast);
    if constexpr (HT * NW == NST && NVB % HT == 0) {
      const int ti0 = w * HT;
#pragma unroll
      for (int i = 0; i < HT; ++i) hacc[i] *= dlast;
      mma_row<T, CH, HT, PT, 1, 1, PT>(hacc, sKdT + 16 * (ti0 / NVB) * PT, sVt + 16 * (ti0 % NVB) * PT);
    } else {
#pragma unroll
      for (int i = 0; i < HT; ++i) {
        const int ti = w * HT + i;
        if (ti < NST) {
          hacc[i] *= dlast;
          mma_tile<T, CH, PT, 1, 1, PT>(hacc[i], sKdT + 16 * (ti / NVB) * PT, sVt + 16 * (ti % NVB) * PT);
        }
      }
    }
    lds_barrier();
    if (!warm) {
      store_rows<T, CH, VD, PK, NT>((T*)p.o + ((long)t0 * p.Hv + h) * VD, (long)p.Hv * VD, sW, len);
      lds_barrier();
    }
  }

  if (write_final && p.ht) {
#pragma unroll
    for (int i = 0; i < HT; ++i) {
      const int ti = w * HT + i, rb = ti / NVB, cb = ti % NVB;
      if (ti < NST) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          p.ht[(((long)n * p.Hv + h) * KD + 16 * rb + acc_row(e)) * VD + 16 * cb + acc_col()] = hacc[i][e];
      }
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
  // persistent grid: three workgroups per CU, each over a contiguous item range
  const long total = (long)p.s.NTtot * p.Hv;
  const int nwg = (int)std::min<long>(padded_grid(total), 3 * 256);
  const int per_wg = (int)((total + nwg - 1) / nwg);
  GDR_LAUNCH("intra_wy", (k_intra<T, KD>), dim3(nwg), st, p, (int)total, per_wg, nwg);
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
  const int total = total_segs * p.Hv;
  timing_before("chunk_fused", st);
  hipLaunchKernelGGL((k_fused<T, KD>), dim3(padded_grid(total)), dim3(512), 0, st, p, total);
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
