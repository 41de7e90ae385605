// gdr_bwd.hip -- backward kernels of the chunked gated delta rule on gfx950.
//
// The backward takes q, k, v, g, beta, (A), do, dht, scale, initial_state and
// returns dq, dk, dv, dbeta, dg, dh0 (FlashQLA curated summary, section
// "使用方式與需求", low-level backward listing); the chunk states are not an
// input, so they are recomputed.  The pages call the backward the hardest part
// of the method, built there as a warp-specialised pipeline under tight
// on-chip memory (same page, section "後向傳播挑戰與warp專屬管線"); here it is
// three passes:
//   1. recompute (forward kernels): g_cum, A, W, U, every chunk's entry state
//      h and Vnew = U - W h;
//   2. k_dstate, serial in reverse over chunks per (sequence, value head,
//      V block): with dh+ the gradient of the state leaving a chunk,
//        dVnew = s P^T dO + diag(e^{gamma_n - gamma}) K dh+
//        dh    = Gamma_n dh+ + s (diag(Gamma) Q)^T dO - W^T dVnew
//      (P = lower(D * Q K^T)); it stores dh+ and dVnew per chunk and dh0;
//   3. k_grads, fully parallel per (chunk, query/key head), looping over the
//      value heads of the group so dq and dk are summed without atomics:
//        dP = s lower(dO Vnew^T),  dQ = dP*D K + s diag(Gamma) dO h^T
//        dW = -dVnew h^T,  dA = lower_strict(dW (b Gamma K)^T + dVnew (b V)^T)
//        dKb = A^T dW,  dVb = A^T dVnew,  dL = lower_strict(-A^T dA A^T)
//        dK = (dP*D)^T Q + (E + E^T) K + diag(b Gamma) dKb
//             + diag(e^{gamma_n - gamma}) Vnew dh+^T,   E = dL * diag(b) D
//        dV = diag(b) dVb,  dbeta and dgamma from the same terms,
//        dg = reverse cumulative sum of dgamma over the chunk.
#include <math.h>
#include <type_traits>

#include "gdr_device.h"
#include "gdr_kernels.h"

namespace gdr {

// -------------------------------------------------------------- k_dstate --
template <typename T, int KD, int BV>
__global__ __launch_bounds__(NTHR) void k_dstate(DStateParams p, int total_items) {
  constexpr int VD = KD;
  constexpr int PK = Pitch<T, KD>::value;
  constexpr int PT = Pitch<T, CH>::value;
  constexpr int PU = Pitch<T, BV>::value;
  constexpr int NCB = BV / 16;
  constexpr int NTILE = (KD / 16) * NCB;
  constexpr int TPW = NTILE / NWAVE;
  static_assert(NTILE % NWAVE == 0, "state tiles must split evenly over the waves");
  __shared__ __align__(16) T sQ[CH * PK];
  __shared__ __align__(16) T sK[CH * PK];
  __shared__ __align__(16) T sQgT[KD * PT];   // s Gamma_t q_t[d]  as [d][t]
  __shared__ __align__(16) T sWnT[KD * PT];   // -W[t][d]          as [d][t]
  __shared__ __align__(16) T sdOT[BV * PT];   // dO[t][v]          as [v][t]
  __shared__ __align__(16) T sPt[CH * PT];    // s P[t][s]         as [s][t]
  __shared__ __align__(16) T sdhT[BV * PK];   // dh+[d][v]         as [v][d]
  __shared__ __align__(16) T sdVT[BV * PT];   // dVnew[t][v]       as [v][t]
  __shared__ __align__(16) T sdVr[CH * PU];   // dVnew rows (global store staging)
  __shared__ __align__(16) T sdhr[KD * PU];   // dh+ rows   (global store staging)
  __shared__ float sG[CH];

  const SeqTables& s = p.s;
  const int u = xcd_remap(blockIdx.x, total_items);
  if (u >= total_items) return;
  const int vb = u % p.nvb;
  const int h = (u / p.nvb) % p.Hv;
  const int n = u / (p.nvb * p.Hv);
  if (n >= s.N) return;
  const int c0 = s.chunk_at(n);
  const int nch = s.chunk_at(n + 1) - c0;
  if (c0 < 0 || nch < 0 || c0 + nch > s.NTtot) return;
  const int hk = h / (p.Hv / p.Hq);
  const int w = wave_id(), l = lane_id();

  f32x4 hacc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int ti = w * TPW + i, rb = ti / NCB, cb = ti % NCB;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int d = 16 * rb + acc_row(e), v = vb * BV + 16 * cb + acc_col();
      hacc[i][e] = p.dht ? p.dht[(((long)n * p.Hv + h) * KD + d) * VD + v] : 0.f;
    }
  }

  TileCols<T, KD> rq, rk, rw;
  TileCols<T, BV> rdo;
  float gam_next = 0.f, glast_next = 0.f;
  auto prefetch = [&](int jc) {  // unconditional; empty range before the first chunk
    const bool valid = jc >= 0;
    const int t0 = s.cu_at(n) + max(jc, 0) * CH;
    const int len = valid ? min(CH, s.cu_at(n + 1) - t0) : 0;
    rq.load((const T*)p.q + ((long)t0 * p.Hq + hk) * KD, (long)p.Hq * KD, len);
    rk.load((const T*)p.k + ((long)t0 * p.Hq + hk) * KD, (long)p.Hq * KD, len);
    rw.load((const T*)p.W + ((long)h * s.Ttot + t0) * KD, KD, len);
    rdo.load((const T*)p.d_o + ((long)t0 * p.Hv + h) * VD + vb * BV, (long)p.Hv * VD, len);
    const rsrc_t gr = make_rsrc(p.gcum + (long)h * s.Ttot + t0, (long)len * 4);
    glast_next = buf_load_f32(gr, (uint32_t)(len - 1) * 4u);
    const float gv = buf_load_f32(gr, (uint32_t)l * 4u);
    gam_next = (l < len) ? gv : glast_next;
  };
  if (nch > 0) prefetch(nch - 1);

  for (int jc = nch - 1; jc >= 0; --jc) {
    const int gc = c0 + jc;
    const int t0 = s.cu_at(n) + jc * CH;
    const int len = min(CH, s.cu_at(n + 1) - t0);
    if (len <= 0 || t0 < 0 || (long)t0 + len > s.Ttot) break;
    const float glast = glast_next, gam = gam_next;
    rq.template store<PK>(sQ);
    rk.template store<PK>(sK);
    rq.template store_t<PT>(sQgT, (l < len) ? p.scale * __expf(gam) : 0.f);
    rw.template store_t<PT>(sWnT, -1.f);
    rdo.template store_t<PT>(sdOT, 1.f);
    if (w == 0) sG[l] = gam;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int ti = w * TPW + i, rb = ti / NCB, cb = ti % NCB;
      acc_store_t<T, PK>(sdhT, 16 * rb, 16 * cb, hacc[i]);
#pragma unroll
      for (int e = 0; e < 4; ++e) sdhr[(16 * rb + acc_row(e)) * PU + 16 * cb + acc_col()] = from_f<T>(hacc[i][e]);
    }
    lds_barrier();
    prefetch(jc - 1);
    store_rows<T, KD, BV, PU>((T*)p.dhbuf + ((long)h * s.NTtot + gc) * KD * VD + vb * BV, VD, sdhr, KD);

    // s P^T as [s][t]: tiles of P = lower(D * Q K^T) with t-block w.
    for (int j = 0; j < 4; ++j) {
      f32x4 a = zero4();
      if (j <= w) {
        mma_tile<T, KD, PK, 1, 1, PK>(a, sQ + 16 * w * PK, sK + 16 * j * PK);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * w + acc_row(e), sidx = 16 * j + acc_col();
          a[e] = (t >= sidx) ? p.scale * __expf(sG[t] - sG[sidx]) * a[e] : 0.f;
        }
      }
      acc_store_t<T, PT>(sPt, 16 * w, 16 * j, a);
    }
    lds_barrier();

    {  // dVnew rows of block w
      f32x4 acc[NCB];
#pragma unroll
      for (int j = 0; j < NCB; ++j) acc[j] = zero4();
      mma_row<T, KD, NCB, PK, 1, 1, PK>(acc, sK + 16 * w * PK, sdhT);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * w + acc_row(e);
        const float dec = (r < len) ? __expf(glast - sG[r]) : 0.f;
#pragma unroll
        for (int j = 0; j < NCB; ++j) acc[j][e] *= dec;
      }
      mma_row<T, CH, NCB, PT, 1, 1, PT>(acc, sPt + 16 * w * PT, sdOT);
#pragma unroll
      for (int j = 0; j < NCB; ++j) {
        acc_store_t<T, PT>(sdVT, 16 * w, 16 * j, acc[j]);
#pragma unroll
        for (int e = 0; e < 4; ++e) sdVr[(16 * w + acc_row(e)) * PU + 16 * j + acc_col()] = from_f<T>(acc[j][e]);
      }
    }
    lds_barrier();
    store_rows<T, CH, BV, PU>((T*)p.dvn + ((long)h * s.Ttot + t0) * VD + vb * BV, VD, sdVr, len);

    const float gl = __expf(glast);
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int ti = w * TPW + i, rb = ti / NCB, cb = ti % NCB;
      hacc[i] *= gl;
      mma_tile<T, CH, PT, 1, 1, PT>(hacc[i], sQgT + 16 * rb * PT, sdOT + 16 * cb * PT);
      mma_tile<T, CH, PT, 1, 1, PT>(hacc[i], sWnT + 16 * rb * PT, sdVT + 16 * cb * PT);
    }
    lds_barrier();
  }

  if (p.dh0) {
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int ti = w * TPW + i, rb = ti / NCB, cb = ti % NCB;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = 16 * rb + acc_row(e), v = vb * BV + 16 * cb + acc_col();
        p.dh0[(((long)n * p.Hv + h) * KD + d) * VD + v] = hacc[i][e];
      }
    }
  }
}

// -------------------------------------------------------------- k_dfused --
// The reverse state pass of the backward, cut into CP segments like the
// forward's fused pass: one 8-wave workgroup per (sequence, value head,
// segment), chunks in reverse order.  Wave w owns state-gradient columns
// 16w..16w+15 over all K rows in fp32 accumulators, rows numbered as in
// k_fused.  Per chunk, with dh the gradient of the state leaving it:
//   kd  = K dh                             (dh as the MFMA B operand)
//   dh <- Gamma_n dh + s (Gamma Q)^T dO    (Q^T by transposing LDS reads)
//   dVn = s P^T dO + dec * kd,  dec_t = e^{gamma_n - gamma_t},  P = lower(D * Q K^T)
//   dh <- dh - W^T dVn = dh - K^T (Gamma * (A''^T dVn)),  W = A'' diag(Gamma) K,
//         A'' = A diag(beta) (staged instead of W, as in the forward)
// and dh entering the chunk (before the update) and dVn are stored for the
// per-chunk gradients.  The dO terms do not depend on dh, so the map from a
// segment's end gradient to its start gradient is affine with the forward
// transition transposed: dh_in = M^T dh_out + d.  A certified head runs each
// segment from up to W warmup chunks after its end, from zero (or from the
// final-state gradient when the window reaches the sequence end); other
// heads run from exact end gradients (k_segscan, reverse mode), and with
// trans = 1 compute the offsets d of their segments from a zero end
// gradient (the last from the final-state gradient).  Q, K, A'', dO and the
// gate cumsums are copied into LDS one chunk ahead as in k_fused; P^T is
// stored with its token columns permuted as k_fused permutes P.
template <typename T>
struct DFusedBufs {   // one buffer of staged chunk inputs
  T *W, *Q, *K, *O;   // W: the A'' tile (64 x 64)
  float *G, *D;       // gate cumsums; per-row factors {e^{gamma_n - gamma_t}, s e^{gamma_t}, e^{gamma_t}}
};

template <int KD, bool TRANS>
__global__ __launch_bounds__(FNT) void k_dfused(DFusedParams p, int total_items) {
  using T = bf16;
  constexpr int VD = KD;
  constexpr int VEC = 8;
  constexpr int NCH = KD / VEC;
  constexpr int TE = CH * KD;
  constexpr int NKB = KD / 16, NCB = VD / 16;
  constexpr int NWV = NCB < FNW ? NCB : FNW;
  static_assert(NCB <= FNW && NKB % 2 == 0, "one column tile per wave, paired row tiles");
  __shared__ __align__(16) T sW0[CH * CH], sQ0[TE], sK0[TE], sO0[TE], sW1[CH * CH], sQ1[TE], sK1[TE], sO1[TE];
  // P^T as a swizzled 64-wide tile (16-byte fragment reads without bank conflicts)
  constexpr int PSZ = CH * CH;
  __shared__ __align__(16) T sP[PSZ];
  __shared__ __align__(16) T sDh[TRANS ? 8 : KD * KD];   // staged dh rows of a chunk
  __shared__ __align__(16) float sG0[CH], sG1[CH], sD0[3 * CH], sD1[3 * CH];
  if (p.Hq < 0) {  // never taken: an ordinary store keeps the copy-only arrays from being folded away
    const T z = from_f<T>(0.f);
    sW0[threadIdx.x] = z; sQ0[threadIdx.x] = z; sK0[threadIdx.x] = z; sO0[threadIdx.x] = z;
    sW1[threadIdx.x] = z; sQ1[threadIdx.x] = z; sK1[threadIdx.x] = z; sO1[threadIdx.x] = z;
    sG0[threadIdx.x & 63] = 0.f; sG1[threadIdx.x & 63] = 0.f;
  }
  auto bufs = [&](auto bc) __attribute__((always_inline)) {
    if constexpr (decltype(bc)::value == 0) return DFusedBufs<T>{sW0, sQ0, sK0, sO0, sG0, sD0};
    else return DFusedBufs<T>{sW1, sQ1, sK1, sO1, sG1, sD1};
  };
  auto tix = [](int r, int c) { return (r * NCH + ((c / VEC) ^ stage_swz<NCH>(r))) * VEC + (c % VEC); };

  const SeqTables& s = p.s;
  int h, item;
  if (!TRANS && s.seg_order) {
    // unequal segments: longest first, head groups round-robin over the XCDs
    // (the forward state passes' order)
    const int G = p.Hv / p.Hq;
    const int x = (int)blockIdx.x & 7, pos = (int)blockIdx.x >> 3;
    const int kg = (pos / G) * 8 + x;
    if (kg >= p.total_segs * p.Hq) return;
    const int r = kg / p.Hq;
    item = s.seg_order[r];
    h = (kg - r * p.Hq) * G + pos % G;
  } else {
    const int u = xcd_remap(blockIdx.x, total_items);
    if (u >= total_items) return;
    h = u % p.Hv;
    item = u / p.Hv;
  }
  const int n = s.seq_of_seg(item);
  const int pseg = item - s.seg_at(n);
  const int nseg = s.seg_at(n + 1) - s.seg_at(n);
  const int c0 = s.chunk_at(n);
  const int nch = s.chunk_at(n + 1) - c0;
  if (pseg < 0 || pseg >= nseg || c0 < 0 || c0 + nch > s.NTtot) return;
  const int seq0 = s.cu_at(n), seq1 = s.cu_at(n + 1);
  const int L = p.seg_chunks;
  const int hk = h / (p.Hv / p.Hq);
  const int w = wave_id(), l = lane_id(), q = l >> 4, t = l & 15, sl = l & 15;
  const bool owner = w < NWV;
  const int col = 16 * w + t;
  const float* hcert = p.cert + (long)h * s.NTtot + c0;
  const int send = min(pseg * L + L, nch);   // the segment's end chunk
  const float wpre = TRANS ? 0.f : warmup_first(hcert, send, 1, nch - send, p.warmup);
  const bool certified = p.hflag ? p.hflag[(long)n * p.Hv + h] != 0
                                 : head_certified(hcert, nseg, nch, L, p.warmup, p.log_eps, true);
  const int gseg = s.seg_at(n) + pseg;
  const long hbase = ((long)n * p.Hv + h) * KD * VD;
  // chunks crs down to cbeg; those below cend are the segment's own
  int cbeg = pseg * L, cend = min(cbeg + L, nch), crs;
  const float* ginit = nullptr;   // end gradient (null: zero)
  if (TRANS) {
    if (certified || pseg == 0) return;
    crs = cend - 1;
    if (pseg == nseg - 1) ginit = p.dht ? p.dht + hbase : nullptr;
  } else if (certified) {
    const int wu = short_warmup(hcert, cend, 1, nch - cend, p.warmup, p.log_eps, wpre);
    crs = min(cend + wu, nch) - 1;
    if (crs == nch - 1) ginit = p.dht ? p.dht + hbase : nullptr;
  } else if (p.dhstart) {
    crs = cend - 1;
    if (pseg == nseg - 1) ginit = p.dht ? p.dht + hbase : nullptr;
    else ginit = p.dhstart + ((long)h * p.total_segs + gseg) * KD * VD;
  } else {
    if (pseg != 0) return;             // segment 0 runs the whole head serially
    cbeg = 0; cend = nch; crs = nch - 1;
    ginit = p.dht ? p.dht + hbase : nullptr;
  }
  auto krow = [&](int rb, int e) { return 32 * (rb >> 1) + 8 * q + 4 * (rb & 1) + e; };
  f32x4 ds[NKB];   // one branch around all the loads, so that they are issued together
#pragma unroll
  for (int rb = 0; rb < NKB; ++rb) ds[rb] = zero4();
  if (owner && ginit) {
#pragma unroll
    for (int rb = 0; rb < NKB; ++rb)
#pragma unroll
      for (int e = 0; e < 4; ++e) ds[rb][e] = ginit[(long)krow(rb, e) * VD + col];
  }

  // Copies of chunk jc's tiles into buffer bc in four parts (0 W, 1 dO, 2 K,
  // 3 Q and the gate cumsums); rows past the chunk read as zero.
  constexpr int NCP = (NCH + FNW - 1) / FNW;
  uint32_t off_qk[NCP], off_o[NCP], off_a[1];
#pragma unroll
  for (int j = 0; j < NCP; ++j) {
    const int i = w + FNW * j;
    const int pidx = 64 * i + l;
    const int r = pidx / NCH, c = (pidx % NCH) ^ stage_swz<NCH>(r);
    off_qk[j] = (uint32_t)(r * p.Hq * KD * (int)sizeof(T) + c * 16);
    off_o[j] = (uint32_t)(r * p.Hv * VD * (int)sizeof(T) + c * 16);
  }
  {  // the 64-wide A'' tile: eight 1 KB blocks, one per wave
    const int pidx = 64 * w + l;
    const int r = pidx >> 3, c = (pidx & 7) ^ stage_swz<8>(r);
    off_a[0] = apack_src(r, c);   // from compact rows
  }
  auto tix8 = [](int r, int c) { return (r * 8 + ((c >> 3) ^ stage_swz<8>(r))) * 8 + (c & 7); };
  auto copy_part = [&](int jc, auto bc, int piece) __attribute__((always_inline)) {
    const DFusedBufs<T> bf = bufs(bc);
    const int t0 = seq0 + jc * CH;
    const int len = min(CH, seq1 - t0);
    const long rbytes = (long)len * KD * (long)sizeof(T);
    if (piece == 0)
      lds_copy_tile<1, 8, FNW, 8, true>(bf.W, rsrc_words((const T*)p.Au + ((long)h * s.Ttot + t0) * CH, apack_bytes(len)), off_a, w);
    if (piece == 1)
      lds_copy_tile<NCP, NCH, FNW, VEC, true>(bf.O, rsrc_words((const T*)p.d_o + ((long)t0 * p.Hv + h) * VD, rbytes * p.Hv), off_o, w);
    if (piece == 2)
      lds_copy_tile<NCP, NCH, FNW, VEC>(bf.K, rsrc_words((const T*)p.k + ((long)t0 * p.Hq + hk) * KD, rbytes * p.Hq), off_qk, w);
    if (piece == 3) {
      lds_copy_tile<NCP, NCH, FNW, VEC>(bf.Q, rsrc_words((const T*)p.q + ((long)t0 * p.Hq + hk) * KD, rbytes * p.Hq), off_qk, w);
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
  // Waits for this wave's copies; wave 0 derives chunk jn's per-row factors;
  // the barrier publishes everything.
  auto wait_copies = [&](int jn, auto bc) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0);
    if (w == 0 && jn >= cbeg) {
      const DFusedBufs<T> bf = bufs(bc);
      const int tn = seq0 + jn * CH;
      const int ln = min(CH, seq1 - tn);
      const float gl = bf.G[max(ln, 1) - 1], gv = bf.G[l];
      bf.D[l] = (l < ln) ? __expf(gl - gv) : 0.f;
      bf.D[CH + l] = p.scale * __expf(gv);
      bf.D[2 * CH + l] = __expf(gv);
      __builtin_amdgcn_s_waitcnt(0xC07F);
    }
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  auto trd = [](const T* a) __attribute__((always_inline)) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)a);
  };

  if (crs >= cbeg) copy_chunk(crs, ic<0>());
  // the upper P tiles (0,1) and (2,3) are always zero: written once here
  // (published by the barrier below), never recomputed
  for (int i = threadIdx.x; i < PSZ; i += FNT) sP[i] = from_f<T>(0.f);
  wait_copies(crs, ic<0>());

  auto step = [&](auto bc, int jc) __attribute__((always_inline)) -> bool {
    constexpr int b = decltype(bc)::value;
    const int t0 = seq0 + jc * CH;
    const int len = min(CH, seq1 - t0);
    if (len <= 0 || t0 < 0 || (long)t0 + len > s.Ttot) return false;
    const bool keep = !TRANS && jc < cend;   // a chunk of the segment itself
    const bool more = jc - 1 >= cbeg;
    const DFusedBufs<T> cur = bufs(bc);
    if (more) {
      copy_part(jc - 1, ic<1 - b>(), 0);
      copy_part(jc - 1, ic<1 - b>(), 1);
    }
    const T* sW = cur.W;
    const T* sQ = cur.Q;
    const T* sK = cur.K;
    const T* sO = cur.O;
    const float* sG = cur.G;
    const float* sD = cur.D;
    const float* sM = cur.D + CH;
    const float glast = sG[len - 1];
    if constexpr (!TRANS) {
      if (keep && owner) {   // gradient of the state leaving the chunk, [K][V] rows
        // 4x4 transposes within lane quads give one 8-byte row piece per lane
        // and tile, staged in LDS; the rows leave as 16-byte pieces after the
        // P^T barrier.
#pragma unroll
        for (int rb = 0; rb < NKB; ++rb)
          *reinterpret_cast<uint2*>(sDh + tix(krow(rb, t & 3), 16 * w + 4 * (t >> 2))) = pack4_bf16(quad_t(ds[rb]));
      }
    }
    {  // P tiles (the ten lower ones; the masked (0,1), (2,3) stay zero from the start), stored transposed
      constexpr int TI[12] = {3, 3, 2, 2, 3, 3, 2, 1, 1, 0, 0, 2};
      constexpr int TJ[12] = {0, 1, 0, 1, 2, 3, 2, 0, 1, 0, 1, 3};
      const int cnt = w < 4 ? 2 : (w < 6 ? 1 : 0);
      int ti[2], tj[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int idx = w < 4 ? 2 * w + m : 8 + (w - 4);
        ti[m] = TI[idx];
        tj[m] = TJ[idx];
      }
      f32x4 pa[2] = {zero4(), zero4()};
      if (cnt > 1) {
#pragma unroll
        for (int k0 = 0; k0 < KD; k0 += 32) {
          bf16x8 fa[2], fb[2];
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            fa[m] = *reinterpret_cast<const bf16x8*>(sQ + tix(16 * ti[m] + t, k0 + 8 * q));
            fb[m] = *reinterpret_cast<const bf16x8*>(sK + tix(16 * tj[m] + t, k0 + 8 * q));
          }
#pragma unroll
          for (int m = 0; m < 2; ++m) pa[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[m], fb[m], pa[m], 0, 0, 0);
        }
      } else if (cnt > 0) {
#pragma unroll
        for (int k0 = 0; k0 < KD; k0 += 32) {
          const bf16x8 fa = *reinterpret_cast<const bf16x8*>(sQ + tix(16 * ti[0] + t, k0 + 8 * q));
          const bf16x8 fb = *reinterpret_cast<const bf16x8*>(sK + tix(16 * tj[0] + t, k0 + 8 * q));
          pa[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb, pa[0], 0, 0, 0);
        }
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        if (m < cnt) {
          // a lane's four rows r0 + e land in four consecutive columns of
          // the stored row c (the permutation keeps r & 3): one 8-byte store
          const int r0 = 16 * ti[m] + 4 * q, c = 16 * tj[m] + t;
          const f32x4 gr = *reinterpret_cast<const f32x4*>(sG + r0);
          const float gc = sG[c];
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (r0 + e >= c && r0 + e < len) ? p.scale * __expf(gr[e] - gc) * pa[m][e] : 0.f;
          const int pr = (r0 & ~31) + 8 * ((r0 >> 2) & 3) + 4 * ((r0 >> 4) & 1);
          *reinterpret_cast<uint2*>(sP + tix8(c, pr)) = pack4_bf16(v);
        }
      }
    }
    if (more) {
      copy_part(jc - 1, ic<1 - b>(), 2);
      copy_part(jc - 1, ic<1 - b>(), 3);
    }
    f32x4 kd[4];
    bf16x8 bo[2];   // dO[32ks + {4q .. 4q+3, 16+4q .. 16+4q+3}][col]
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) kd[tt] = zero4();
    if (owner) {
#pragma unroll
      for (int ks = 0; ks < KD / 32; ++ks) {   // kd = K dh
        bf16x8 ak[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) ak[tt] = *reinterpret_cast<const bf16x8*>(sK + tix(16 * tt + t, 32 * ks + 8 * q));
        const bf16x8 hb = pack_b(ds[2 * ks], ds[2 * ks + 1]);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) kd[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak[tt], hb, kd[tt], 0, 0, 0);
      }
      const float gn = __expf(glast);
#pragma unroll
      for (int rb = 0; rb < NKB; ++rb) ds[rb] *= gn;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {   // dh += s (Gamma Q)^T dO
        const int ra = 32 * ks + 4 * q + (sl >> 2);
        bo[ks] = cat4(trd(sO + tix(ra, 16 * w + 4 * (sl & 3))), trd(sO + tix(ra + 16, 16 * w + 4 * (sl & 3))));
        const f32x4 mlo = *reinterpret_cast<const f32x4*>(sM + 32 * ks + 4 * q);
        const f32x4 mhi = *reinterpret_cast<const f32x4*>(sM + 32 * ks + 16 + 4 * q);
        bf16x8 by;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16 xl = bo[ks][i], xh = bo[ks][4 + i];
          by[i] = from_f<T>(to_f(xl) * mlo[i]);
          by[4 + i] = from_f<T>(to_f(xh) * mhi[i]);
        }
#pragma unroll
        for (int rb = 0; rb < NKB; ++rb) {
          const int cc = 32 * (rb >> 1) + 8 * (sl & 3) + 4 * (rb & 1);
          const bf16x8 aq = cat4(trd(sQ + tix(ra, cc)), trd(sQ + tix(ra + 16, cc)));
          ds[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, by, ds[rb], 0, 0, 0);
        }
      }
    }
    lds_barrier();   // P^T complete
    if constexpr (!TRANS) {
      if (keep) {   // the staged dh rows to memory
        T* db = (T*)p.dhbuf + ((long)h * s.NTtot + c0 + jc) * KD * VD;
#pragma unroll
        for (int i = threadIdx.x; i < KD * NCH; i += FNT) {
          const int r = i / NCH, c = i % NCH;
          *reinterpret_cast<uint4*>(db + (long)r * VD + c * VEC) =
              *reinterpret_cast<const uint4*>(sDh + (r * NCH + (c ^ stage_swz<NCH>(r))) * VEC);
        }
      }
    }
    if (owner) {
      f32x4 dv[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) dv[tt] = zero4();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)   // s P^T dO: row tile tt needs tokens >= 16 tt
#pragma unroll
        for (int tt = 0; tt <= 2 * ks + 1; ++tt) {
          const bf16x8 ap = *reinterpret_cast<const bf16x8*>(sP + tix8(16 * tt + t, 32 * ks + 8 * q));
          dv[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ap, bo[ks], dv[tt], 0, 0, 0);
        }
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) dv[tt][e] += sD[16 * tt + acc_row(e)] * kd[tt][e];
      if (keep) {   // dVn token rows, 8-byte row pieces after quad transposes
        T* vb = (T*)p.dvn + ((long)h * s.Ttot + t0) * VD + 16 * w + 4 * (t >> 2);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const uint2 u = pack4_bf16(quad_t(dv[tt]));
          const int r = 16 * tt + 4 * q + (t & 3);
          if (r < len) *reinterpret_cast<uint2*>(vb + (long)r * VD) = u;
        }
      }
      // z = Gamma * (A''^T dVn), rows s in blocks st (A'' lower triangular)
      f32x4 z[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) z[st] = zero4();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 bv = pack_b(dv[2 * ks], dv[2 * ks + 1]);
        const int ra = 32 * ks + 4 * q + (sl >> 2);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          if (2 * ks + 1 >= st) {
            const int cs = 16 * st + 4 * (sl & 3);
            const bf16x8 aa = cat4(trd(sW + tix8(ra, cs)), trd(sW + tix8(ra + 16, cs)));
            z[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aa, bv, z[st], 0, 0, 0);
          }
        }
      }
      const float* sGa = sD + 2 * CH;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const f32x4 ga = *reinterpret_cast<const f32x4*>(sGa + 16 * st + 4 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) z[st][e] *= -ga[e];
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {   // dh -= K^T z
        const int ra = 32 * ks + 4 * q + (sl >> 2);
        const bf16x8 bz = pack_b(z[2 * ks], z[2 * ks + 1]);
#pragma unroll
        for (int rb = 0; rb < NKB; ++rb) {
          const int cc = 32 * (rb >> 1) + 8 * (sl & 3) + 4 * (rb & 1);
          const bf16x8 ak = cat4(trd(sK + tix(ra, cc)), trd(sK + tix(ra + 16, cc)));
          ds[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, bz, ds[rb], 0, 0, 0);
        }
      }
    }
    wait_copies(jc - 1, ic<1 - b>());   // the next chunk's tiles have landed; P^T is free again
    return true;
  };
  for (int jc = crs; jc >= cbeg; jc -= 2) {
    if (!step(ic<0>(), jc) || jc - 1 < cbeg || !step(ic<1>(), jc - 1)) break;
  }

  if (owner) {
    float* dst = nullptr;
    if (TRANS) dst = p.segtr + (((long)h * p.total_segs + gseg) * 2 + 1) * KD * VD;
    else if (cbeg == 0 && p.dh0) dst = p.dh0 + hbase;
    if (dst) {
#pragma unroll
      for (int rb = 0; rb < NKB; ++rb)
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[(long)krow(rb, e) * VD + col] = ds[rb][e];
    }
  }
}

// --------------------------------------------------------------- k_grads --
// LDS: permanent K rows, K^T and Q^T; three 64-row regions R1..R3 and four
// 64x64 tiles S0..S3 whose contents change phase by phase (see comments).
template <typename T, int KD>
__global__ __launch_bounds__(NTHR) void k_grads(GradParams p) {
  constexpr int VD = KD;
  constexpr int PK = Pitch<T, KD>::value;
  constexpr int PT = Pitch<T, CH>::value;
  constexpr int PL = 68;
  constexpr int NKT = KD / 16;
  constexpr int NVT = VD / 16;
  constexpr int SZ_R = ((CH * PK > KD * PT ? CH * PK : KD * PT) * (int)sizeof(T) > CH * PL * 4)
                           ? (CH * PK > KD * PT ? CH * PK : KD * PT) * (int)sizeof(T)
                           : CH * PL * 4;
  constexpr int SZ_S = CH * PT * (int)sizeof(T);
  static_assert(2 * SZ_S >= CH * PK * (int)sizeof(T), "S2+S3 must hold 64 value rows");
  __shared__ __align__(16) T sK[CH * PK];
  __shared__ __align__(16) T sKT[KD * PT];
  __shared__ __align__(16) T sQT[KD * PT];
  __shared__ __align__(16) char rbuf[3 * SZ_R + 4 * SZ_S];
  __shared__ float sG[CH], sB[CH], sGm[CH], sDec[CH], sdg[CH], sdb[CH];
  __shared__ float colp[NWAVE][CH];
  __shared__ float red[2][NWAVE];
  T* R1 = reinterpret_cast<T*>(rbuf);
  T* R2 = reinterpret_cast<T*>(rbuf + SZ_R);
  T* R3 = reinterpret_cast<T*>(rbuf + 2 * SZ_R);
  T* S0 = reinterpret_cast<T*>(rbuf + 3 * SZ_R);
  T* S1 = reinterpret_cast<T*>(rbuf + 3 * SZ_R + SZ_S);
  T* S2 = reinterpret_cast<T*>(rbuf + 3 * SZ_R + 2 * SZ_S);
  T* S3 = reinterpret_cast<T*>(rbuf + 3 * SZ_R + 3 * SZ_S);

  const SeqTables& s = p.s;
  const int total = s.NTtot * p.Hq;
  const int u = xcd_remap(blockIdx.x, total);
  if (u >= total) return;
  const int c = u / p.Hq, hk = u % p.Hq;
  int n, t0, len;
  if (!locate_chunk_b(s, c, n, t0, len)) return;
  const int G = p.Hv / p.Hq;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();

  // group-shared tiles: K rows, K^T, Q^T; raw Q K^T and K K^T (row block w)
  f32x4 Sqk[4], Skk[4];
  {
    TileCols<T, KD> rq, rk;
    rq.load((const T*)p.q + ((long)t0 * p.Hq + hk) * KD, (long)p.Hq * KD, len);
    rk.load((const T*)p.k + ((long)t0 * p.Hq + hk) * KD, (long)p.Hq * KD, len);
    rq.template store<PK>(R1);
    rk.template store<PK>(sK);
    rq.template store_t<PT>(sQT, 1.f);
    rk.template store_t<PT>(sKT, 1.f);
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j) { Sqk[j] = zero4(); Skk[j] = zero4(); }
  mma_row<T, KD, 4, PK, 1, 1, PK>(Sqk, R1 + 16 * w * PK, sK);
  mma_row<T, KD, 4, PK, 1, 1, PK>(Skk, sK + 16 * w * PK, sK);
  f32x4 dq[NKT], dk[NKT];
#pragma unroll
  for (int j = 0; j < NKT; ++j) { dq[j] = zero4(); dk[j] = zero4(); }
  __syncthreads();

  for (int gi = 0; gi < G; ++gi) {
    const int h = hk * G + gi;
    const long hT = (long)h * s.Ttot;
    // ---- ph1: per-head rows and scalars
    float glast;
    {
      const float* gc = p.gcum + hT + t0;
      glast = gc[len - 1];
      if (w == 0) {
        const float gm = (l < len) ? gc[l] : glast;
        sG[l] = gm;
        sB[l] = (l < len) ? p.beta[(long)(t0 + l) * p.Hv + h] : 0.f;
        sGm[l] = (l < len) ? __expf(gm) : 0.f;
        sDec[l] = (l < len) ? __expf(glast - gm) : 0.f;
        sdg[l] = 0.f;
        sdb[l] = 0.f;
      }
      colp[w][l] = 0.f;
    }
    TileCols<T, VD> rdvn, rv;
    {
      TileCols<T, VD> rdo, rvn;
      rdo.load((const T*)p.d_o + ((long)t0 * p.Hv + h) * VD, (long)p.Hv * VD, len);
      rvn.load((const T*)p.vnew + (hT + t0) * VD, VD, len);
      rdvn.load((const T*)p.dvn + (hT + t0) * VD, VD, len);
      rv.load((const T*)p.v + ((long)t0 * p.Hv + h) * VD, (long)p.Hv * VD, len);
      TileCols<float, CH> ra;   // A rows (fp32): row-major -> S0, transposed -> S1
      ra.load(p.A_ws + (hT + t0) * CH, CH, len);
#pragma unroll
      for (int i = 0; i < TileCols<float, CH>::NV; ++i) {
        const int c0 = (w + NWAVE * i) * 4;
        const float* e = reinterpret_cast<const float*>(&ra.v[i]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          S0[l * PT + c0 + j] = from_f<T>(e[j]);
          S1[(c0 + j) * PT + l] = from_f<T>(e[j]);
        }
      }
      rdo.template store<PK>(R1);
      rvn.template store<PK>(R2);
      rdvn.template store<PK>(R3);
    }
    lds_barrier();

    // ---- ph2: dP (regs), dQ_inter, dW (regs), dKhat; gate terms
    f32x4 dP[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) dP[j] = zero4();
    mma_row<T, VD, 4, PK, 1, 1, PK>(dP, R1 + 16 * w * PK, R2);
    float rowx[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float colx = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * w + acc_row(e), sidx = 16 * j + acc_col();
        const float D = (t >= sidx) ? __expf(sG[t] - sG[sidx]) : 0.f;
        const float dpd = p.scale * dP[j][e] * D;
        const float x = dpd * Sqk[j][e];
        dP[j][e] = dpd;                // now (dP * D)
        rowx[e] += x;
        colx += x;
      }
      colx = col_group_sum(colx);
      if (l < 16) colp[w][16 * j + l] -= colx;
    }

    const T* hb = (const T*)p.hbuf + ((long)h * s.NTtot + c) * KD * VD;    // [d][v]
    const T* dhb = (const T*)p.dhbuf + ((long)h * s.NTtot + c) * KD * VD;  // [d][v]
    f32x4 aw[NKT];
    {
      f32x4 aq[NKT];
#pragma unroll
      for (int j = 0; j < NKT; ++j) { aq[j] = zero4(); aw[j] = zero4(); }
      constexpr int KS = Mma<T>::KSTEP;
#pragma unroll
      for (int k0 = 0; k0 < VD; k0 += KS) {
        const auto fdo = Mma<T>::template load<PK, 1>(R1 + 16 * w * PK + k0);
        const auto fdv = Mma<T>::template load<PK, 1>(R3 + 16 * w * PK + k0);
#pragma unroll
        for (int j = 0; j < NKT; ++j) {
          const auto fh = Mma<T>::template load<VD, 1>(hb + 16 * j * VD + k0);
          aq[j] = Mma<T>::op(fdo, fh, aq[j]);
          aw[j] = Mma<T>::op(fdv, fh, aw[j]);
        }
      }
      // dQ_inter = s Gamma_t (dO h^T)_t ; dgamma_t += <q_t, dQ_inter_t>
      float qd[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * w + acc_row(e);
        const float sc = p.scale * sGm[t];
#pragma unroll
        for (int j = 0; j < NKT; ++j) {
          const float v = sc * aq[j][e];
          dq[j][e] += v;
          qd[e] += v * to_f(sQT[(16 * j + acc_col()) * PT + t]);
          aw[j][e] = -aw[j][e];        // dW = -dVnew h^T
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) rowx[e] += qd[e];   // per-lane partial, reduced at the end
    }
    {
      // dKhat = Vnew dh+^T; dK += diag(dec) dKhat; r_t = <k_t, dec_t dKhat_t>
      f32x4 ak[NKT];
#pragma unroll
      for (int j = 0; j < NKT; ++j) ak[j] = zero4();
      float hd = 0.f;
      constexpr int KS = Mma<T>::KSTEP;
#pragma unroll
      for (int k0 = 0; k0 < VD; k0 += KS) {
        const auto fvn = Mma<T>::template load<PK, 1>(R2 + 16 * w * PK + k0);
#pragma unroll
        for (int j = 0; j < NKT; ++j) {
          const auto fdh = Mma<T>::template load<VD, 1>(dhb + 16 * j * VD + k0);
          ak[j] = Mma<T>::op(fvn, fdh, ak[j]);
          if (w == 0) {  // <dh+, h> over the whole state, once
            const auto fh = Mma<T>::template load<VD, 1>(hb + 16 * j * VD + k0);
            if constexpr (std::is_same<T, float>::value) {
              hd += fh * fdh;
            } else {
#pragma unroll
              for (int q = 0; q < 8; ++q) hd += to_f(fh[q]) * to_f(fdh[q]);
            }
          }
        }
      }
      float rk[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * w + acc_row(e);
        const float dec = sDec[t];
#pragma unroll
        for (int j = 0; j < NKT; ++j) {
          const float v = dec * ak[j][e];
          dk[j][e] += v;
          rk[e] += v * to_f(sK[t * PK + 16 * j + acc_col()]);
        }
      }
      float rsum = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        rowx[e] -= rk[e];                              // per-lane partial
        rsum += rk[e];
      }
      rsum = wave_sum(rsum);
      hd = wave_sum(hd);
      if (l == 0) { red[0][w] = rsum; red[1][w] = (w == 0) ? hd : 0.f; }
    }
    lds_barrier();

    // ---- ph3: dW rows -> R1, dW^T -> R2, value rows -> S2..S3
#pragma unroll
    for (int j = 0; j < NKT; ++j) {
#pragma unroll
      for (int e = 0; e < 4; ++e) R1[(16 * w + acc_row(e)) * PK + 16 * j + acc_col()] = from_f<T>(aw[j][e]);
      acc_store_t<T, PT>(R2, 16 * w, 16 * j, aw[j]);
    }
    rv.template store<PK>(S2);
    lds_barrier();

    // ---- ph4: dA (strict lower) and dKb = A^T dW
    f32x4 dA[4];
    {
      f32x4 ta[4], tb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) { ta[j] = zero4(); tb[j] = zero4(); }
      mma_row<T, KD, 4, PK, 1, 1, PK>(ta, R1 + 16 * w * PK, sK);
      mma_row<T, VD, 4, PK, 1, 1, PK>(tb, R3 + 16 * w * PK, S2);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * w + acc_row(e), sidx = 16 * j + acc_col();
          dA[j][e] = (t > sidx) ? sB[sidx] * (sGm[sidx] * ta[j][e] + tb[j][e]) : 0.f;
        }
    }
    {
      f32x4 akb[NKT];
#pragma unroll
      for (int j = 0; j < NKT; ++j) akb[j] = zero4();
      mma_row<T, CH, NKT, PT, 1, 1, PT>(akb, S1 + 16 * w * PT, R2);
      float kk[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * w + acc_row(e);
        const float bg = sB[t] * sGm[t];
#pragma unroll
        for (int j = 0; j < NKT; ++j) {
          dk[j][e] += bg * akb[j][e];
          kk[e] += akb[j][e] * to_f(sK[t * PK + 16 * j + acc_col()]);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * w + acc_row(e);
        rowx[e] += sB[t] * sGm[t] * kk[e];              // per-lane partial
        const float ks = row_group_sum(kk[e]);          // <dKb_t, k_t>
        if (acc_col() == 0) sdb[t] += sGm[t] * ks;
      }
    }
    lds_barrier();

    // ---- ph5: dVnew^T -> R1, dA^T -> R2
    rdvn.template store_t<PT>(R1, 1.f);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc_store_t<T, PT>(R2, 16 * w, 16 * j, dA[j]);
    lds_barrier();

    // ---- ph6: dVb = A^T dVnew -> dv (staged in R3); M1 = A^T dA
    f32x4 m1[4];
    {
      f32x4 av[NVT];
#pragma unroll
      for (int j = 0; j < NVT; ++j) av[j] = zero4();
      mma_row<T, CH, NVT, PT, 1, 1, PT>(av, S1 + 16 * w * PT, R1);
      float vv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * w + acc_row(e);
        const float b = sB[t];
#pragma unroll
        for (int j = 0; j < NVT; ++j) {
          vv[e] += av[j][e] * to_f(S2[t * PK + 16 * j + acc_col()]);
          R3[t * PK + 16 * j + acc_col()] = from_f<T>(b * av[j][e]);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float vs = row_group_sum(vv[e]);
        if (acc_col() == 0) sdb[16 * w + acc_row(e)] += vs;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) m1[j] = zero4();
      mma_row<T, CH, 4, PT, 1, 1, PT>(m1, S1 + 16 * w * PT, R2);
    }
    lds_barrier();
    store_rows<T, CH, VD, PK>((T*)p.dv + ((long)t0 * p.Hv + h) * VD, (long)p.Hv * VD, R3, len);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) S2[(16 * w + acc_row(e)) * PT + 16 * j + acc_col()] = from_f<T>(m1[j][e]);
    lds_barrier();

    // ---- ph8: dL = strict_lower(-M1 A^T); E = dL * diag(b) D; gate/beta terms
    float* E32 = reinterpret_cast<float*>(R1);
    {
      f32x4 dl[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) dl[j] = zero4();
      mma_row<T, CH, 4, PT, 1, 1, PT>(dl, S2 + 16 * w * PT, S0);
      float bsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float colx = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * w + acc_row(e), sidx = 16 * j + acc_col();
          float ev = 0.f;
          if (t > sidx) {
            const float D = __expf(sG[t] - sG[sidx]);
            const float dlv = -dl[j][e];
            const float y = dlv * D * Skk[j][e];
            bsum[e] += y;
            ev = dlv * sB[t] * D;
            const float x = sB[t] * y;
            rowx[e] += x;
            colx += x;
          }
          E32[t * PL + sidx] = ev;
        }
        colx = col_group_sum(colx);
        if (l < 16) colp[w][16 * j + l] -= colx;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float bs = row_group_sum(bsum[e]);
        if (acc_col() == 0) sdb[16 * w + acc_row(e)] += bs;
      }
    }
    // (dP * D) rows -> R2, its transpose -> S3
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int e = 0; e < 4; ++e) R2[(16 * w + acc_row(e)) * PT + 16 * j + acc_col()] = from_f<T>(dP[j][e]);
      acc_store_t<T, PT>(S3, 16 * w, 16 * j, dP[j]);
    }
    // row-sum gate terms of this wave's rows
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float rs = row_group_sum(rowx[e]);
      if (acc_col() == 0) sdg[16 * w + acc_row(e)] += rs;
    }
    lds_barrier();
    // F = E + E^T -> S1
    for (int i = tid; i < CH * CH; i += NTHR) {
      const int r = i / CH, cc = i % CH;
      S1[r * PT + cc] = from_f<T>(E32[r * PL + cc] + E32[cc * PL + r]);
    }
    lds_barrier();

    // ---- ph9: dQ += (dP*D) K; dK += (dP*D)^T Q + F K
    mma_row<T, CH, NKT, PT, 1, 1, PT>(dq, R2 + 16 * w * PT, sKT);
    mma_row<T, CH, NKT, PT, 1, 1, PT>(dk, S3 + 16 * w * PT, sQT);
    mma_row<T, CH, NKT, PT, 1, 1, PT>(dk, S1 + 16 * w * PT, sKT);

    // gate: dgamma_t = row terms - column terms (+ last-row terms); dg is its
    // reverse cumulative sum over the chunk's tokens.
    if (w == 0) {
      float dgm = sdg[l] + colp[0][l] + colp[1][l] + colp[2][l] + colp[3][l];
      if (l == len - 1) {
        const float rs = red[0][0] + red[0][1] + red[0][2] + red[0][3];
        dgm += rs + __expf(glast) * red[1][0];
      }
      dgm = (l < len) ? dgm : 0.f;
      // suffix sum: scan over reversed lanes
      const float rev = __shfl(dgm, 63 - l, 64);
      const float sc = wave_inclusive_scan(rev);
      const float dgv = __shfl(sc, 63 - l, 64);
      if (l < len) {
        p.dg[(long)(t0 + l) * p.Hv + h] = dgv;
        p.dbeta[(long)(t0 + l) * p.Hv + h] = sdb[l];
      }
    }
    lds_barrier();
  }

  // dq, dk rows -> LDS -> global
#pragma unroll
  for (int j = 0; j < NKT; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      R1[(16 * w + acc_row(e)) * PK + 16 * j + acc_col()] = from_f<T>(dq[j][e]);
      R2[(16 * w + acc_row(e)) * PK + 16 * j + acc_col()] = from_f<T>(dk[j][e]);
    }
  __syncthreads();
  store_rows<T, CH, KD, PK>((T*)p.dq + ((long)t0 * p.Hq + hk) * KD, (long)p.Hq * KD, R1, len);
  store_rows<T, CH, KD, PK>((T*)p.dk + ((long)t0 * p.Hq + hk) * KD, (long)p.Hq * KD, R2, len);
}

// ------------------------------------------------------------- launchers --
static unsigned padded_grid_b(long total) { return (unsigned)(((total + 7) / 8) * 8); }

template <typename T, int KD, int BV>
static hipError_t dstate_impl(const DStateParams& p, int total, hipStream_t st) {
  timing_before("chunk_dstate", st);
  hipLaunchKernelGGL((k_dstate<T, KD, BV>), dim3(padded_grid_b(total)), dim3(NTHR), 0, st, p, total);
  hipError_t err = hipGetLastError();
  timing_after(st);
  return err;
}

template <typename T, int KD>
static hipError_t grads_impl(const GradParams& p, hipStream_t st) {
  timing_before("chunk_grads", st);
  hipLaunchKernelGGL((k_grads<T, KD>), dim3(padded_grid_b((long)p.s.NTtot * p.Hq)), dim3(NTHR), 0, st, p);
  hipError_t err = hipGetLastError();
  timing_after(st);
  return err;
}

hipError_t launch_dstate(DType dt, int KD, int BV, const DStateParams& p, int total, hipStream_t st) {
  if (dt == DType::BF16) {
    if (KD == 32 && BV == 32) return dstate_impl<bf16, 32, 32>(p, total, st);
    if (KD == 64 && BV == 32) return dstate_impl<bf16, 64, 32>(p, total, st);
    if (KD == 128 && BV == 64) return dstate_impl<bf16, 128, 64>(p, total, st);
  } else {
    if (KD == 32 && BV == 32) return dstate_impl<float, 32, 32>(p, total, st);
    if (KD == 64 && BV == 32) return dstate_impl<float, 64, 32>(p, total, st);
  }
  return hipErrorInvalidValue;
}

template <int KD>
static hipError_t dfused_impl(const DFusedParams& p, int total_segs, hipStream_t st) {
  const int total = total_segs * p.Hv;
  if (!p.trans && p.s.seg_order && (total_segs > 1024 || total_segs != p.total_segs)) return hipErrorInvalidValue;
  // with a segment order: 8 XCDs x G slots per round of head groups
  const unsigned grid = (!p.trans && p.s.seg_order)
      ? (unsigned)(8 * (p.Hv / p.Hq) * (((long)total_segs * p.Hq + 7) / 8)) : padded_grid_b(total);
  timing_before(p.trans ? "cp_rev_transition" : "chunk_dfused", st);
  if (p.trans) hipLaunchKernelGGL((k_dfused<KD, true>), dim3(grid), dim3(FNT), 0, st, p, total);
  else hipLaunchKernelGGL((k_dfused<KD, false>), dim3(grid), dim3(FNT), 0, st, p, total);
  hipError_t err = hipGetLastError();
  timing_after(st);
  return err;
}

hipError_t launch_dfused(DType dt, int KD, const DFusedParams& p, int total_segs, hipStream_t st) {
  if (dt != DType::BF16) return hipErrorInvalidValue;
  if (KD == 32) return dfused_impl<32>(p, total_segs, st);
  if (KD == 64) return dfused_impl<64>(p, total_segs, st);
  if (KD == 128) return dfused_impl<128>(p, total_segs, st);
  return hipErrorInvalidValue;
}

hipError_t launch_grads(DType dt, int KD, const GradParams& p, hipStream_t st) {
  if (dt == DType::BF16) {
    if (KD == 32) return grads_impl<bf16, 32>(p, st);
    if (KD == 64) return grads_impl<bf16, 64>(p, st);
    if (KD == 128) return grads_impl<bf16, 128>(p, st);
  } else {
    if (KD == 32) return grads_impl<float, 32>(p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdr
