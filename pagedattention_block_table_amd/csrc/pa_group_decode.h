// Grouped decode for batches whose sequences share prefix blocks.
//
// Pages (by title and section):
//   [P3] "内存优化：KV Cache管理、PagedAttention原理与内存池配置" — prefix caching: requests
//        with the same system prompt map it to the same physical blocks (reference counted),
//        64 requests of 1000 tokens sharing ~500 of them in the worked case;
//   [P1] "突破GPU内存瓶颈：vLLM与PagedAttention技术深度解析" §2 / §5 — block tables map
//        logical to physical blocks and several sequences may name the same block.
//
// What is computed is exactly pa_decode's result (attention of each sequence's query heads
// over its own cached tokens); only the reading changes. A workgroup takes one KV head g
// and a group of NG = 16 / G consecutive sequences (G query heads per KV head), whose 16
// query rows (row rho = member rho / G, head rho % G) fill the 16 columns of the transposed
// matrix-core engine (S^T = K Q^T, O^T += V^T P^T; see MfmaTEngine). The group's tokens are
// walked in 16-token chunks by logical position. For each chunk the members' table entries
// are compared: every distinct physical block gives one pass, which loads that block's 16
// K and V rows once and updates the rows of every member that maps the chunk to it (the
// other rows are masked: their scores are -inf, their probabilities exactly 0, so their
// state does not change). A prefix block shared by the whole group is therefore read once
// for the group instead of once per sequence, and private blocks once each, as before.
//
// A row sees its sequence's chunks in the same order whatever the sharing: the order of
// arithmetic depends only on logical positions, so shared and privately copied prefixes
// give the same bits (the lazy max raise is decided per row, matrix-core columns are
// independent, and a masked row's update adds exact zeros).
//
// Work split: the chunks of a (KV head, group) are dealt to nsplit workgroups (chunk c to
// split c mod nsplit) and, within one, to its waves round robin. Each wave builds the list
// of its passes for 64 chunks at a time in LDS (one lane per chunk: member ids and
// validity, distinct blocks, a wave prefix sum for the offsets), then runs them with the
// next pass's loads in flight. At the end the waves merge through LDS; with one split the
// workgroup writes the outputs, else it writes (max, exp-sum, partial output) per (sequence,
// head, split) and the log-sum-exp merge kernel combines the splits.
#pragma once

namespace pa {

#ifndef PA_GROUP_ROTATE
#define PA_GROUP_ROTATE 1
#endif
constexpr bool kGroupRotate = PA_GROUP_ROTATE != 0;

template <int IO, int KV, int D, int BS, int G, int NW, bool DBG>
struct GroupShape {
  static constexpr int NG = 16 / G;  // sequences per group
  using Geo = MfmaGeo<KV, D>;
  static constexpr int RB = Geo::RB;
  static constexpr int TILE_BYTES = BS * RB;
  static constexpr int NDT = D / 16;
  static constexpr int NV = VTileRegs<KV, D>::NV;
  static constexpr int VT_ROW = D + 16;
  static constexpr int VT_BYTES = 16 * VT_ROW * 2;
  static constexpr int KT_ROW = RB + 16;  // bytes per K row staged in the V tile's LDS
  static constexpr int MAXP = 64 * NG;  // passes of one window of 64 chunks
  static constexpr int PVT = KV == kBF16 ? kBF16 : kF16;
  static constexpr bool SPLIT_P = PVT == kBF16;
  struct WaveLds {
    char vt[VT_BYTES];
    int2 pass[MAXP];
  };
  static constexpr int LOOP_BYTES = NW * (int)sizeof(WaveLds);
  static constexpr int MERGE_BYTES = NW * 16 * (D + 2) * 4;
  static constexpr int LDS_BYTES = LOOP_BYTES > MERGE_BYTES ? LOOP_BYTES : MERGE_BYTES;
  static constexpr bool ok = (G == 2 || G == 4 || G == 8) && BS >= 16 && mfma_supported<IO, KV, D, G>();
  static_assert(!ok || 16 * KT_ROW <= VT_BYTES, "K tile fits the V tile's LDS");
};

// Registers of one pass in flight: the lane's share of the chunk's K rows and of its V
// rows, both in memory order (instruction i, lane l: bytes 1024 i + 16 l of the chunk's 16
// rows), plus the pass's chunk start, member mask and load bound.
template <int KV, int D>
struct GroupBuf {
  uint4 kr[MfmaGeo<KV, D>::CPL];
  VTileRegs<KV, D> vt;
  int c0, mask, lmax, bid;
};

template <int IO, int KV, int D, int BS, int G, int NW, bool DBG>
__global__ void __launch_bounds__(NW * 64) grouped_decode_kernel(const DecodeArgs a) {
  using Sh = GroupShape<IO, KV, D, BS, G, NW, DBG>;
  static_assert(Sh::ok, "unsupported grouped decode shape");
  constexpr int NG = Sh::NG, RB = Sh::RB, NDT = Sh::NDT, NV = Sh::NV, VT_ROW = Sh::VT_ROW;
  using Geo = MfmaGeo<KV, D>;
  using M16 = Mma16<Sh::PVT>;
  using v4 = typename M16::v4;
  using elem = typename M16::elem;
  using vec = typename Mma<IO>::vec;
  using Buf = GroupBuf<KV, D>;
  using WaveLds = typename Sh::WaveLds;

  __shared__ __align__(16) char lds[Sh::LDS_BYTES];

  const int S = a.num_seqs;
  const int H = a.num_heads;
  // decode: a group is NG consecutive sequences; short queries (extend): a group is one
  // sequence and member i is its new token i, at position L - Q + i, attending over
  // positions 0 .. L - Q + i through the sequence's one block table
  const bool ext = a.query_start_loc != nullptr;
  const int ngroups = ext ? S : (S + NG - 1) / NG;
  const int nsplit = a.num_parts;
  const int unit = xcd_unit((int)blockIdx.x, (int)gridDim.x);
  const int q = unit % nsplit;
  const int gg = unit / nsplit;  // KV-head major: gg = g * ngroups + group
  const int grp = gg % ngroups;
  const int g = gg / ngroups;
  const int s0 = ext ? grp : grp * NG;
  int q0 = 0, Qs = 0;
  if (ext) {
    q0 = a.query_start_loc[grp];
    Qs = a.query_start_loc[grp + 1] - q0;
    if (Qs <= 0 || Qs > NG) return;  // whole workgroup: not a short query
  }
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const LaneIds li(tid & 63);
  const int rho = li.n;  // this lane's query row: member rho / G, head rho % G
  const int mi = rho / G;

  // members' context lengths (uniform), the lane's own, and the group's longest
  int Lm[NG];
  int Lmax = 0;
  const int Lseq = ext ? min(max(a.context_lens[s0], 0), a.max_ctx) : 0;
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    if (ext)
      Lm[i] = i < Qs ? min(max(Lseq - Qs + i + 1, 0), a.max_ctx) : 0;
    else
      Lm[i] = s0 + i < S ? min(max(a.context_lens[s0 + i], 0), a.max_ctx) : 0;
    Lmax = max(Lmax, Lm[i]);
  }
  int L_own = 0;
#pragma unroll
  for (int i = 0; i < NG; ++i) L_own = mi == i ? Lm[i] : L_own;
  // the query row of this lane: sequence s_own (decode) or new token q0 + mi (extend)
  const int64_t s_own = ext ? (int64_t)q0 + min(mi, Qs - 1) : (int64_t)min(s0 + mi, S - 1);

  const int nch = (Lmax + 15) / 16;                                  // chunks of the group
  const int nk = nch > q ? (nch - q + nsplit - 1) / nsplit : 0;      // chunks of this split
  const int nwk = wave < nk ? (nk - wave + NW - 1) / NW : 0;         // chunks of this wave
  // groups start their walk at evenly spread chunks, so that the workgroups of a shared
  // prefix do not all load the same block at the same moment (the order depends only on
  // the group index and its length, never on where the blocks live)
  const int rot = kGroupRotate && nch > 0 ? (int)((int64_t)grp * nch / ngroups) : 0;
  auto chunk_of = [&](int kk) { return rotated(q + nsplit * (wave + NW * kk), rot, nch); };

  // query operand: row rho's head, the same k order as the K rows of the lanes' loads
  vec qa[Geo::NST];
  {
    const uint16_t* qrow = (const uint16_t*)a.q + (s_own * H + g * G + rho % G) * D;
#pragma unroll
    for (int i = 0; i < Geo::CPL; ++i) {
      const int col = Geo::VEC * (4 * i + li.lg);
#pragma unroll
      for (int hf = 0; hf < Geo::VEC / 8; ++hf)
        qa[i * (Geo::VEC / 8) + hf] = __builtin_bit_cast(vec, *(const uint4*)(qrow + col + 8 * hf));
    }
  }
  float m = -3.0e38f, l = 0.f;
  f32x4_t o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  WaveLds& wl = ((WaveLds*)lds)[wave];
  const int64_t blk_stride = (int64_t)a.num_kv_heads * Sh::TILE_BYTES;
  const char* kbase = (const char*)a.k_pool + (int64_t)g * Sh::TILE_BYTES;
  const char* vbase = (const char*)a.v_pool + (int64_t)g * Sh::TILE_BYTES;
  const int32_t* bt0 = a.block_tables + (int64_t)s0 * a.max_blocks_per_seq;
  const int MB = a.max_blocks_per_seq;
  const int mstride = ext ? 0 : MB;  // table row of member i: bt0 + i * mstride
  int w0 = 0;  // first chunk of the current window (in this wave's chunk order)

  // pass p of the current window: the loads of its chunk from its block (live = false:
  // not consumed, every lane reads the chunk's first row)
  auto issue = [&](Buf& b, int p, bool live) {
    const int2 d = wl.pass[p];
    const int bid = min(max(__builtin_amdgcn_readfirstlane(d.x), 0), a.num_blocks - 1);
    const int dy = __builtin_amdgcn_readfirstlane(d.y);
    const int mask = dy & 0xffff;
    const int c = chunk_of(w0 + (dy >> 16));
    const int c0 = 16 * c;
    int lmax = 0;
#pragma unroll
    for (int i = 0; i < NG; ++i) lmax = (mask >> i) & 1 ? max(lmax, Lm[i]) : lmax;
    b.c0 = c0;
    b.mask = mask;
    b.lmax = lmax;
    b.bid = bid;
    const char* kb = kbase + (int64_t)bid * blk_stride;
    const char* vb = vbase + (int64_t)bid * blk_stride;
    // rows at or past every member's context end read the chunk's first row instead
    // (finite data of this block; those rows are masked for every member). K, like V, in
    // whole 1 KiB runs of the chunk's 16 contiguous rows (put into the MFMA layout through
    // LDS when consumed)
    const int lim = live ? lmax : 0;
    const char* kchunk = kb + (c0 % BS) * RB;
#pragma unroll
    for (int i = 0; i < Geo::CPL; ++i) {
      const int byte = 1024 * i + 16 * li.lane;
      b.kr[i] = load16(kchunk + (c0 + byte / RB < lim ? byte : byte % RB));
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int byte = 1024 * i + 16 * li.lane;
      int t = c0 + byte / RB;
      t = t < lim ? t : c0;
      b.vt.v[i] = load16(vb + (t % BS) * RB + byte % RB);
    }
  };

  auto consume = [&](const Buf& b, int) {
    const int c0 = b.c0;
    const int mask = b.mask;
    if constexpr (DBG) {
      // one load of 16 rows of block b.bid (KV head g), whatever the number of members
      if (a.dbg_block_reads && li.lane == 0)
        atomicAdd(a.dbg_block_reads + (int64_t)b.bid * a.num_kv_heads + g, 1);
      // each member of the pass consumes these rows: copy them and count the reads
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        if (!((mask >> i) & 1)) continue;
        const int64_t row0 = ((int64_t)(s0 + i) * a.num_kv_heads + g) * a.dbg_max_ctx;
#pragma unroll
        for (int k = 0; k < Geo::CPL; ++k) {
          const int byte = 1024 * k + 16 * li.lane;
          const int t = c0 + byte / RB;
          if (t < Lm[i]) {
            *(uint4*)((char*)a.dbg_k + (row0 + t) * RB + byte % RB) = b.kr[k];
            if (byte % RB == 0) atomicAdd(a.dbg_counts + row0 + t, 1);
          }
        }
#pragma unroll
        for (int k = 0; k < NV; ++k) {
          const int byte = 1024 * k + 16 * li.lane;
          const int t = c0 + byte / RB;
          if (t < Lm[i]) *(uint4*)((char*)a.dbg_v + (row0 + t) * RB + byte % RB) = b.vt.v[k];
        }
      }
    }
    // the previous pass's transposed reads come before these writes
    MfmaTEngine<IO, KV, D, BS, G, 1, DBG>::lds_exchange();
    // K into the MFMA layout (lane (n, lg): row n, chunks 4i + lg) through the tile,
    // read back before V overwrites it
    uint4 kr[Geo::CPL];
#pragma unroll
    for (int i = 0; i < Geo::CPL; ++i) {
      const int byte = 1024 * i + 16 * li.lane;
      *(uint4*)(wl.vt + (byte / RB) * Sh::KT_ROW + byte % RB) = b.kr[i];
    }
    MfmaTEngine<IO, KV, D, BS, G, 1, DBG>::lds_exchange();
#pragma unroll
    for (int i = 0; i < Geo::CPL; ++i) kr[i] = *(const uint4*)(wl.vt + li.n * Sh::KT_ROW + 16 * (4 * i + li.lg));
    MfmaTEngine<IO, KV, D, BS, G, 1, DBG>::lds_exchange();
    uint16_t* vt = (uint16_t*)wl.vt;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int byte = 1024 * i + 16 * li.lane;
      const int t = byte / RB;
      const int col = (byte % RB) / ElemBytes<KV>::value;
      if constexpr (KV == kFP8) {
        const uint4 r = b.vt.v[i];
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
        uint32_t packed[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          packed[2 * k] = fp8x2_to_mt<Sh::PVT, false>(w[k]);
          packed[2 * k + 1] = fp8x2_to_mt<Sh::PVT, true>(w[k]);
        }
        *(uint4*)(vt + t * VT_ROW + col) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
        *(uint4*)(vt + t * VT_ROW + col + 8) = make_uint4(packed[4], packed[5], packed[6], packed[7]);
      } else {
        *(uint4*)(vt + t * VT_ROW + col) = b.vt.v[i];
      }
    }
    MfmaTEngine<IO, KV, D, BS, G, 1, DBG>::lds_exchange();

    // this lane's row takes part in the pass if its member maps the chunk to this block
    const int t_end = (mask >> mi) & 1 ? L_own : 0;
    f32x4_t cs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < Geo::CPL; ++i)
#pragma unroll
      for (int hf = 0; hf < Geo::VEC / 8; ++hf)
        cs = Mma<IO>::mma(k_operand<IO, KV>(kr[i], hf), qa[i * (Geo::VEC / 8) + hf], cs);
    float z[4];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      z[r] = c0 + 4 * li.lg + r < t_end ? cs[r] * a.q_mul : -INFINITY;
      mx = fmaxf(mx, z[r]);
    }
    mx = rows4_max(mx);
    const bool raise = mx > m + kLazyRescale;
    if (__any(raise)) {
      const float mn = raise ? mx : m;
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      m = mn;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[dt][r] *= alpha;
    }
    v4 phi, plo;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = __builtin_amdgcn_exp2f(z[r] - m);
      l += p;
      if constexpr (Sh::SPLIT_P) {
        uint16_t hi, lo;
        M16::split(p, hi, lo);
        phi[r] = __builtin_bit_cast(elem, hi);
        plo[r] = __builtin_bit_cast(elem, lo);
      } else {
        phi[r] = (_Float16)p;
      }
    }
    const int vrow = 4 * li.lg + (li.n >> 2);
    const int vcol = 4 * (li.n & 3);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const v4 av = __builtin_bit_cast(
          v4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (__attribute__((address_space(3))) i16x4_t*)(vt + vrow * VT_ROW + 16 * dt + vcol)));
      o[dt] = M16::mma(av, phi, o[dt]);
      if constexpr (Sh::SPLIT_P) o[dt] = M16::mma(av, plo, o[dt]);
    }
  };

  // windows of 64 of this wave's chunks: build the pass list, then run it
  struct Runner {
    using Buf = GroupBuf<KV, D>;
    decltype(issue)& iss;
    decltype(consume)& con;
    __device__ __forceinline__ void issue(const DecodeArgs&, Buf& b, int k, bool live) { iss(b, k, live); }
    __device__ __forceinline__ void consume(const DecodeArgs&, const Buf& b, int k) { con(b, k); }
  };
  for (; w0 < nwk; w0 += 64) {
    const int kk = w0 + li.lane;
    const bool live = kk < nwk;
    const int c = live ? chunk_of(kk) : 0;
    int bid[NG];
    bool val[NG];
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      val[i] = live && 16 * c < Lm[i];
      bid[i] = val[i] ? bt0[(int64_t)i * mstride + (16 * c) / BS] : -1;
    }
    // a pass for each member whose block no earlier member of the chunk maps it to
    bool lead[NG];
    int np = 0;
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      bool first = val[i];
#pragma unroll
      for (int j = 0; j < i; ++j) first = first && !(val[j] && bid[j] == bid[i]);
      lead[i] = first;
      np += first ? 1 : 0;
    }
    int incl = np;
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) {
      const int y = __shfl_up(incl, k);
      if (li.lane >= k) incl += y;
    }
    const int total = __builtin_amdgcn_readlane(incl, 63);
    int p = incl - np;
    // the previous window's passes have all been consumed (in order) before this rewrite
    MfmaTEngine<IO, KV, D, BS, G, 1, DBG>::lds_exchange();
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      if (lead[i]) {
        int mask = 0;
#pragma unroll
        for (int j = i; j < NG; ++j) mask |= (val[j] && bid[j] == bid[i]) ? 1 << j : 0;
        wl.pass[p] = make_int2(bid[i], (li.lane << 16) | mask);
        ++p;
      }
    }
    MfmaTEngine<IO, KV, D, BS, G, 1, DBG>::lds_exchange();
    Runner run{issue, consume};
    run_pipelined(run, a, total);
  }

  // merge the waves' row states through LDS (reusing the loop's LDS) and write
  __syncthreads();
  float* sm_o = (float*)lds;                 // [NW][16][D]
  float* sm_m = sm_o + NW * 16 * D;          // [NW][16]
  float* sm_l = sm_m + NW * 16;              // [NW][16]
  const float lt = rows4_sum(l);
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) sm_o[(wave * 16 + rho) * D + 16 * dt + 4 * li.lg + r] = o[dt][r];
  if (li.lg == 0) {
    sm_m[wave * 16 + rho] = m;
    sm_l[wave * 16 + rho] = lt;
  }
  __syncthreads();
  const int64_t NPH = (int64_t)S * H * nsplit;
  for (int idx = tid; idx < 16 * D; idx += NW * 64) {
    const int row = idx / D;
    const int d = idx % D;
    const int s = s0 + row / G;
    if (ext ? row / G >= Qs : s >= S) continue;
    // output row: the member's sequence (decode) or its new token (extend)
    const int64_t orow = ext ? (int64_t)q0 + row / G : (int64_t)s;
    float Mx = sm_m[row];
#pragma unroll
    for (int w = 1; w < NW; ++w) Mx = fmaxf(Mx, sm_m[w * 16 + row]);
    float ov = 0.f, lsum = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = __builtin_amdgcn_exp2f(sm_m[w * 16 + row] - Mx);
      ov = fmaf(f, sm_o[(w * 16 + row) * D + d], ov);
      lsum = fmaf(f, sm_l[w * 16 + row], lsum);
    }
    const int h = g * G + row % G;
    if (nsplit == 1) {
      store_io<IO>(a.out, (orow * H + h) * D + d, lsum > 0.f ? (ov / lsum) * a.out_mul : 0.f);
    } else {
      const int64_t slot = ((int64_t)s * H + h) * nsplit + q;
      a.ws[2 * NPH + slot * D + d] = ov * a.out_mul;
      if (d == 0) {
        a.ws[slot] = Mx;
        a.ws[NPH + slot] = lsum;
      }
    }
  }
}

}  // namespace pa
