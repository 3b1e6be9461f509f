// flk_attn.hip -- single-token grouped-query decode attention read straight from packed K/V
// chains (FlashLoop RFC, vllm-rlt #156, section 3.3: optimized readers consume the packed
// base/residual tiles during QK and PV instead of keeping a BF16 shadow cache).
//
// Every wave works alone on a run of 64-token tiles of one KV head, 16 tokens (one MFMA
// slice) at a time, with no block barrier until the end:
//   1. per tile it scatters each compact loop's rows of the tile (found with the tile index)
//      into a wave-private position -> compact-row map, and stages the tile's K parameter rows
//      in wave-private LDS;
//   2. it decodes K_hat of the slice bit for bit as the encoder left it, straight into the A
//      operand registers of S^T = K_hat Q^T (v_mfma_f32_16x16x32_bf16): a lane's A operand is
//      8 consecutive channels of one token, which is exactly one decode item;
//   3. it keeps an online softmax per query head in binary32;
//   4. it decodes V_hat of the slice into a wave-private LDS tile and accumulates
//      O^T += V_hat^T P^T with v_mfma_f32_16x16x16_bf16, whose P^T operand layout is the score
//      tile's register layout, so probabilities never leave registers.
// At the end the block's 4 waves merge their (m, l, O) through LDS into one partial per
// (block, query head); a second kernel merges the partials of all blocks.  A BF16 tail (a
// rolling cache's recent tokens) is read as stored, 16 tokens per wave.
#include <mutex>

#include "flk_attn_common.h"

// The partials buffer of flk_decode_attn_packed_noalloc, for callers that cannot allocate: one
// copy per GPU, held until the process ends, shared by every such call on that GPU.  Host code
// never passes this name to a kernel (on the host it is only a stand-in for the symbol); it uses
// the device address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[FLK_NOALLOC_SCRATCH_BYTES];

namespace flk {

// The workspace a call over T packed tokens and a tail of tail_len tokens uses: one partial
// (m, l, O) and one block maximum per query head and split, then the two-pass path's scores,
// one row of ceil(T/4)*4 binary32 per query head (T counting the tail's tokens as well).
static size_t attn_ws_bytes(int32_t splits, int32_t T, int32_t Hq) {
  return size_t(splits) * size_t(Hq) * (2 + kAttnD + 1) * sizeof(float) +
         size_t(Hq) * ((size_t(T) + 3) & ~size_t(3)) * sizeof(float);
}
// (Sized with the one-pass reader's split count, which the two-pass reader's never exceeds.)
size_t attn_workspace_need(int32_t T, int32_t tail_len, int32_t H, int32_t Hq) {
  return attn_ws_bytes(n_splits(attn_tiles(T, tail_len), H), T + tail_len, Hq);
}

// A bound on attn_workspace_need for every call over at most T_total tokens: such a call has at
// most ceil(T_total/64) + 1 tiles (a packed prefix and a tail may each end in a partial tile),
// the split count does not decrease with the tile count, and the packed part is at most T_total.
size_t attn_workspace_bytes(int32_t T_total, int32_t H, int32_t Hq) {
  const int64_t tiles = (int64_t(T_total) + kGroup - 1) / kGroup + 1;
  const int32_t s = n_splits(int32_t(tiles < INT32_MAX ? tiles : INT32_MAX), H);
  return attn_ws_bytes(s, T_total, Hq);
}

// SC: also write every (query head, packed token) scaled score to scores[head][position], rows
// of ceil(T/4)*4 floats (the reference loop of sparse decode attention selects keys from them).
template <int NL, bool SC, int FMT = 0>
__global__ __launch_bounds__(kAThreads, FLK_ATTN_OCC) void attn_wave_kernel(ChainArgs kc, ChainArgs vc, int32_t T, int32_t H,
                                                              int32_t G, const uint16_t* __restrict__ q,
                                                              const uint16_t* __restrict__ kt,
                                                              const uint16_t* __restrict__ vt, int32_t tail_len,
                                                              float scale, int32_t wph,
                                                              float* __restrict__ ws_ml, float* __restrict__ ws_o,
                                                              float* __restrict__ scores) {
  __shared__ __attribute__((aligned(16))) unsigned char s_raw[attn_lds_bytes<NL>()];
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int n = lane & 15;                                // MFMA column: query head / token / channel
  const int kb = lane >> 4;                               // MFMA k-block / row block
  // Blocks are renumbered split-major, head-minor, and each XCD runs a contiguous range of the
  // new numbers: the H heads of a token range run together in one L2.  A token's codes of heads
  // 2m and 2m+1 share a 128-byte line, and a row's V parameters of all heads share one, so
  // those lines are fetched once instead of once per head.
  const uint32_t lin = xcd_remap(blockIdx.x + blockIdx.y * gridDim.x, gridDim.x * gridDim.y);
  const int32_t split = int32_t(lin / gridDim.y);
  const int32_t h = int32_t(lin % gridDim.y);
  const int32_t Hq = H * G;
  const int32_t ptiles = (T + kGroup - 1) / kGroup;       // packed tiles
  // the head's packed tiles, ptiles / wph per wave and one more for the first ptiles % wph
  const int32_t w = split * kAWaves + wave;               // this wave's index within its head
  const int32_t base = ptiles / wph, extra = ptiles - base * wph;
  const int32_t tile0 = w < wph ? w * base + min(w, extra) : ptiles;
  const int32_t tile1 = w < wph ? tile0 + base + (w < extra ? 1 : 0) : ptiles;
  WaveLds<NL>& L = reinterpret_cast<WaveLds<NL>*>(s_raw)[wave];

  // Q^T as the B operand of S^T = K_hat Q^T: lane holds Q[n][32*ks + 8*kb + j], zero past G
  bf16x8_t qb[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    uint4 w = make_uint4(0, 0, 0, 0);
    if (n < G) w = *reinterpret_cast<const uint4*>(q + int64_t(h * G + n) * kAttnD + 32 * ks + 8 * kb);
    qb[ks] = __builtin_bit_cast(bf16x8_t, w);
  }
  // decode items of this lane: token n of the slice, octets 4*i + kb (the K A-operand layout)
  int oc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) oc[i] = 4 * i + kb;

  // NVFP4 loops: the stream scales, loaded once (kept out of the tile loop, where their scalar
  // loads would share a wait counter with the LDS reads of the K parameter rows)
  float sgk[NL], sgv[NL];
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    sgk[l] = loop_nv<FMT>(l) && l < kc.n_loops ? __uint_as_float(kc.s[l].params[0]) : 0.0f;
    sgv[l] = loop_nv<FMT>(l) && l < vc.n_loops ? __uint_as_float(vc.s[l].params[0]) : 0.0f;
  }

  float m_run = -__builtin_inff(), l_run = 0.0f;
  float4_t o[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) o[mt] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  // INT4 V loops go to the MFMA as codes (VNIB): the A operand is 1024 + code in binary16, the B
  // operand p * scale per token and V group, so the products carry 1024 * sum(B) on top of
  // sum(code * B).  vmin accumulates, per V group, the minimum's share sum(p * min) minus that
  // 1024 * sum(B) over this lane's tokens; it is added to every channel of the group at the end.
  // Other formats decode V_hat to BF16 first (exact).
  constexpr bool VNIB = FMT == 0;
  float vmin[2] = {0.0f, 0.0f};

  // Exact PV of one slice: V_hat (this lane: token n, octets oc[]) through wave-private LDS into
  // the A operands, p as BF16.
  auto pv_exact = [&](const uint4 (&vitem)[4], const float (&p)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(&L.v[n][oc[i] * 8]) = vitem[i];
    wave_sync();
    short4_t pb;
#pragma unroll
    for (int j = 0; j < 4; ++j) pb[j] = short(__builtin_bit_cast(uint16_t, (__bf16)p[j]));
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      short4_t a;
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = short(L.v[4 * kb + j][pv_channel(mt, n)]);
      o[mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb, o[mt], 0, 0, 0);
    }
    wave_sync();                                          // the slice's V reads before the next writes
  };

  // One 16-token slice: S^T = K_hat Q^T on the MFMA (kitem: the A operands), one online-softmax
  // step, then the PV products (vpath, given this lane's 4 probabilities).  Slots 4*kb + i at or
  // past nv are masked.
  auto attend_slice = [&](const uint4 (&kitem)[4], int32_t nv, auto&& vpath, auto&& emit) {
    float4_t sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kitem[ks]), qb[ks], sacc, 0, 0, 0);
    // online softmax; lane holds the scores of tokens 4*kb + i of the slice for head n
    float sc[4];
    float mx = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[i] = 4 * kb + i < nv ? sacc[i] * scale : -__builtin_inff();
      mx = fmaxf(mx, sc[i]);
    }
    emit(sc);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    float p[4], psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = m_new == -__builtin_inff() ? 0.0f : __expf(sc[i] - m_new);
      psum += p[i];
    }
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    const float corr = m_run == -__builtin_inff() ? 0.0f : __expf(m_run - m_new);
    l_run = l_run * corr + psum;
    m_run = m_new;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) o[mt] = o[mt] * corr;
    if constexpr (VNIB) {
      vmin[0] *= corr;
      vmin[1] *= corr;
    }
    vpath(p);
  };

  // The BF16 tail, read as stored, in 16-token slices: slice s goes to waves s, s + wph, ...
  // of every head, a small addition to many waves rather than whole tiles for a few.
  const int32_t tail_slices = (tail_len + 15) / 16;
  for (int32_t ts = w; w < wph && ts < tail_slices; ts += wph) {
    const int32_t nv = min(16, tail_len - 16 * ts);
    const bool ok = n < nv;
    const int64_t b = (int64_t(16 * ts + n) * H + h) * kAttnD;
    uint4 item[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      item[i] = ok ? *reinterpret_cast<const uint4*>(kt + b + oc[i] * 8) : make_uint4(0, 0, 0, 0);
    attend_slice(item, nv, [&](const float (&p)[4]) {
      uint4 v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        v[i] = ok ? *reinterpret_cast<const uint4*>(vt + b + oc[i] * 8) : make_uint4(0, 0, 0, 0);
      pv_exact(v, p);
    }, [](const float (&)[4]) {});
  }

  for (int32_t tile = tile0; tile < tile1; ++tile) {
    const int32_t t0 = tile * kGroup;
    const TileRows<NL> rk = tile_rows<NL>(kc, tile, T);
    const TileRows<NL> rv = tile_rows<NL>(vc, tile, T);
    wave_sync();                                          // the previous tile's LDS reads are done
    build_maps<NL>(kc, rk, t0, L.map[0], lane);
    build_maps<NL>(vc, rv, t0, L.map[1], lane);
    // K parameter rows of the tile: rowgroup lo/64 (and lo/64 + 1 for a compact loop), each in
    // the slot of its parity, so a row j finds its parameters in slot (j/64) & 1; with tile
    // groups, the tile's own row in slot 0
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      if (l >= kc.n_loops || loop_fp4<FMT>(l)) continue;    // FP4 loops carry no K parameter rows
      if (kc.ktile) {
        if (rk.hi[l] > rk.lo[l]) {
          const uint2 w = *reinterpret_cast<const uint2*>(kc.s[l].params + (uint32_t(tile) * uint32_t(H) + uint32_t(h)) * kAttnD + 2 * lane);
          *reinterpret_cast<uint2*>(&L.kp[l][0][2 * lane]) = w;
        }
        continue;
      }
      const int32_t nrg = (kc.s[l].n + kGroup - 1) / kGroup;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int32_t rg = rk.lo[l] / kGroup + r;
        if ((r == 1 && rk.dense[l]) || rg >= nrg) continue;
        const uint2 w = *reinterpret_cast<const uint2*>(kc.s[l].params + (uint32_t(rg) * uint32_t(H) + uint32_t(h)) * kAttnD + 2 * lane);
        *reinterpret_cast<uint2*>(&L.kp[l][rg & 1][2 * lane]) = w;
      }
    }
    // Order the tile's positions so that positions listed by the same loops sit together (the
    // softmax sum does not depend on the order): a 16-token slice then mostly holds one loop
    // pattern, and a loop none of its tokens has is skipped by the whole wave.  Positions past
    // T go last.  Groups are ranked in order of first occurrence.
    const int32_t n_valid = min(kGroup, T - t0);
    {
      uint32_t key = 0;
#pragma unroll
      for (int l = 1; l < NL; ++l) {
        if (l < kc.n_loops && !rk.dense[l] && L.map[0][l][lane] >= 0) key |= 1u << l;
        if (l < vc.n_loops && !rv.dense[l] && L.map[1][l][lane] >= 0) key |= 1u << (NL + l);
      }
      const bool valid = lane < n_valid;
      const uint64_t below = (uint64_t(1) << lane) - 1;
      uint64_t remaining = __ballot(valid);
      int base = 0, rank = 0;
      while (remaining) {
        const int leader = __builtin_ctzll(remaining);
        const uint32_t k = __builtin_amdgcn_readlane(key, leader);
        const uint64_t grp = __ballot(valid && key == k);
        if (valid && key == k) rank = base + __builtin_popcountll(grp & below);
        base += __builtin_popcountll(grp);
        remaining &= ~grp;
      }
      if (!valid) rank = lane;                              // the invalid tail keeps its order
      L.perm[rank] = lane;
    }
    wave_sync();

    for (int sl = 0; sl * 16 < n_valid; ++sl) {
      const int tk = L.perm[16 * sl + n];
      // VNIB: the slice's INT4 V codes and parameters of every loop are copied into the wave's
      // LDS staging by buffer loads that write LDS directly (no registers held), issued before
      // the K decode so their latency hides behind K's.  Lane L copies 16 bytes of code row
      // L / 4 (chunk vchunk) and, for L < 32, parameter word L % 2 of row L / 2.  A row the loop
      // does not list (or past T) reads zeros, which contribute nothing; a loop none of the
      // slice's rows has is skipped.
      uint32_t vlive = 0;
      if constexpr (VNIB) {
        const int crow = lane >> 2, prow = (lane & 31) >> 1;
        const int cq = (lane & 3) ^ ((crow >> 2) & 3);     // the chunk this lane's slot holds
        const int ctk = L.perm[16 * sl + crow], ptk = L.perm[16 * sl + prow];
        wave_sync();                                          // the previous slice's staging is read
#pragma unroll
        for (int l = 0; l < NL; ++l) {
          if (l >= vc.n_loops) continue;
          const int32_t tc = t0 + ctk, tp = t0 + ptk;
          const int32_t jc = rv.dense[l] ? (tc < T ? tc : -1) : L.map[1][l][ctk];
          const int32_t jp = rv.dense[l] ? (tp < T ? tp : -1) : L.map[1][l][ptk];
          if (__ballot(jc >= 0) == 0) continue;
          vlive |= 1u << l;
          const uint32_t nb = uint32_t(vc.s[l].n) * uint32_t(H);
          const BufRsrc cb = make_buf(vc.s[l].codes, nb * (kAttnD / 2));
          const BufRsrc pb = make_buf(vc.s[l].params, nb * 8u);
          const uint32_t co = jc >= 0 ? (uint32_t(jc) * uint32_t(H) + uint32_t(h)) * (kAttnD / 2) + 16u * uint32_t(cq)
                                      : kOutOfRange;
          const uint32_t po = lane < 32 && jp >= 0 ? (uint32_t(jp) * uint32_t(H) + uint32_t(h)) * 8u + 4u * uint32_t(lane & 1)
                                                   : kOutOfRange;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(cb, (lds_ptr_t)&L.vs.codes[l][0][0], 16, co, 0, 0, 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(pb, (lds_ptr_t)&L.vs.params[l][0], 4, po, 0, 0, 0);
        }
      }
      // K_hat of the slice straight into the A operands
      uint4 item[4];
      decode_items<FLK_KIND_K, NL, FMT>(kc, rk, t0, T, H, h, tk, oc, L.map[0], L.kp, sgk, item);
      attend_slice(item, n_valid - 16 * sl, [&](const float (&p)[4]) {
        if constexpr (VNIB) {
          // B operands: p * scale16 per V group, rows (0, 1) and (2, 3) as binary16 pairs; the
          // minimum's share p * min16 accumulates in binary32 (dot2).  A operands: output tile
          // mt takes nibble mt of each row's word, as binary16 1024 + code.
          const uint32_t pp01 = pack_f16x2(p[0], p[1]), pp23 = pack_f16x2(p[2], p[3]);
          const f16x2_t m1024 = __builtin_bit_cast(f16x2_t, 0xE400E400u);   // (-1024, -1024)
          __builtin_amdgcn_s_waitcnt(0x0F70);                 // vmcnt(0): the staging has landed
          wave_sync();
#pragma unroll
          for (int l = 0; l < NL; ++l) {
            if (!((vlive >> l) & 1u)) continue;
            // this lane's rows 4*kb + r: the 16-bit words at bytes 2n and 32 + 2n, and the row's
            // two parameter words
            uint32_t d[4];
            uint2 vpw[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int row = 4 * kb + r;
              const uint16_t* cr = reinterpret_cast<const uint16_t*>(&L.vs.codes[l][row][0]);
              const uint32_t lo = cr[(16 * vchunk(row, n >> 3) + ((2 * n) & 15)) >> 1];
              const uint32_t hi = cr[(16 * vchunk(row, 2 + (n >> 3)) + ((2 * n) & 15)) >> 1];
              d[r] = lo | (hi << 16);
              vpw[r] = *reinterpret_cast<const uint2*>(&L.vs.params[l][2 * row]);
            }
            f16x4_t bg[2];
#pragma unroll
            for (int g = 0; g < 2; ++g) {
              const uint32_t w0 = g ? vpw[0].y : vpw[0].x, w1 = g ? vpw[1].y : vpw[1].x;
              const uint32_t w2 = g ? vpw[2].y : vpw[2].x, w3 = g ? vpw[3].y : vpw[3].x;
              const uint32_t s01 = __builtin_amdgcn_perm(w1, w0, 0x07060302u), s23 = __builtin_amdgcn_perm(w3, w2, 0x07060302u);
              const uint32_t m01 = __builtin_amdgcn_perm(w1, w0, 0x05040100u), m23 = __builtin_amdgcn_perm(w3, w2, 0x05040100u);
              const f16x2_t b01 = __builtin_bit_cast(f16x2_t, pp01) * __builtin_bit_cast(f16x2_t, s01);
              const f16x2_t b23 = __builtin_bit_cast(f16x2_t, pp23) * __builtin_bit_cast(f16x2_t, s23);
              bg[g] = f16x4_of(__builtin_bit_cast(uint32_t, b01), __builtin_bit_cast(uint32_t, b23));
              vmin[g] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pp01), __builtin_bit_cast(f16x2_t, m01), vmin[g], false);
              vmin[g] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pp23), __builtin_bit_cast(f16x2_t, m23), vmin[g], false);
              vmin[g] = __builtin_amdgcn_fdot2(b01, m1024, vmin[g], false);
              vmin[g] = __builtin_amdgcn_fdot2(b23, m1024, vmin[g], false);
            }
            const uint32_t e0 = d[0] >> 4, e1 = d[1] >> 4, e2 = d[2] >> 4, e3 = d[3] >> 4;
            const uint32_t nib = opaque(0x000F000Fu);           // a VGPR operand: one v_and_or per word
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) {
              const uint32_t b = uint32_t(mt >> 1);
              const uint32_t sel = b | 0x0C00u | ((4u + b) << 16) | 0x0C000000u;   // [x0.b, 0, x1.b, 0]
              const uint32_t x01 = (mt & 1) ? __builtin_amdgcn_perm(e1, e0, sel) : __builtin_amdgcn_perm(d[1], d[0], sel);
              const uint32_t x23 = (mt & 1) ? __builtin_amdgcn_perm(e3, e2, sel) : __builtin_amdgcn_perm(d[3], d[2], sel);
              const f16x4_t a = f16x4_of((x01 & nib) | 0x64006400u, (x23 & nib) | 0x64006400u);
              o[mt] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, bg[mt >> 2], o[mt], 0, 0, 0);
            }
          }
        } else {
          uint4 v[4];
          decode_items<FLK_KIND_V, NL, FMT>(vc, rv, t0, T, H, h, tk, oc, L.map[1], L.kp, sgv, v);
          pv_exact(v, p);
        }
      }, [&](const float (&sc)[4]) {
        if constexpr (SC) {
          if (n < G) {
            float* row = scores + int64_t(h * G + n) * ((int64_t(T) + 3) & ~int64_t(3)) + t0;  // rows padded to 16 B
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int slot = 16 * sl + 4 * kb + i;
              if (slot < n_valid) row[L.perm[slot]] = sc[i];
            }
          }
        }
      });
    }
  }

  if constexpr (VNIB) {
    // the minimum's share and the offset: over the 4 k-blocks, every lane then holds its head's
    float vm[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      vm[g] = vmin[g] + __shfl_xor(vmin[g], 16);
      vm[g] += __shfl_xor(vm[g], 32);
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[mt][i] += vm[mt >> 2];
  }

  // merge the 4 waves: (m, l) per head and O^T per (head, channel) through LDS
  __syncthreads();
  float* s_m = reinterpret_cast<float*>(s_raw);           // [4][16]
  float* s_l = s_m + kAWaves * kMaxG;                     // [4][16]
  float* s_o = s_l + kAWaves * kMaxG;                     // [4][16][128]
  if (kb == 0) {
    s_m[wave * kMaxG + n] = m_run;
    s_l[wave * kMaxG + n] = l_run;
  }
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_o[(wave * kMaxG + n) * kAttnD + pv_channel(mt, 4 * kb + i)] = o[mt][i];
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * kAttnD; idx += kAThreads) {
    const int g = idx / kAttnD, ch = idx % kAttnD;
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kAWaves; ++w) M = fmaxf(M, s_m[w * kMaxG + g]);
    float Ls = 0.0f, O = 0.0f;
#pragma unroll
    for (int w = 0; w < kAWaves; ++w) {
      const float mw = s_m[w * kMaxG + g];
      const float f = mw == -__builtin_inff() ? 0.0f : __expf(mw - M);
      Ls += s_l[w * kMaxG + g] * f;
      O += s_o[(w * kMaxG + g) * kAttnD + ch] * f;
    }
    const int64_t qi = int64_t(split) * Hq + h * G + g;
    if (ch == 0) { ws_ml[2 * qi] = M; ws_ml[2 * qi + 1] = Ls; }
    ws_o[qi * kAttnD + ch] = O;
  }
}

// Merge the per-block partials of one query head over one range of 16 channels: block
// (blockIdx.x = query head, blockIdx.y = channel range); thread (c = tid % 16, g = tid / 16)
// takes channel c of every kCombGroups-th split from g on, with independent loads in flight;
// the groups then merge through LDS.  Every block finds the global maximum itself.
constexpr int kCombGroups = 16;
constexpr int kCombChannels = 16;
constexpr int kCombThreads = kCombGroups * kCombChannels;
__global__ __launch_bounds__(kCombThreads) void attn_combine_kernel(int32_t splits, int32_t Hq,
                                                                   const float* __restrict__ ws_ml,
                                                                   const float* __restrict__ ws_o,
                                                                   uint16_t* __restrict__ out,
                                                                   float* __restrict__ out32,
                                                                   float* __restrict__ ml_out) {
  __shared__ float s_red[kCombThreads];
  __shared__ float s_l[kCombThreads];
  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  const int c = int(blockIdx.y) * kCombChannels + tid % kCombChannels, g = tid / kCombChannels;
  // global maximum of the partial maxima
  float M = -__builtin_inff();
  for (int s = tid; s < splits; s += kCombThreads) M = fmaxf(M, ws_ml[2 * (int64_t(s) * Hq + i)]);
  s_red[tid] = M;
  __syncthreads();
  for (int w = kCombThreads / 2; w > 0; w >>= 1) {
    if (tid < w) s_red[tid] = fmaxf(s_red[tid], s_red[tid + w]);
    __syncthreads();
  }
  M = s_red[0];
  __syncthreads();
  float L = 0.0f, O = 0.0f;
#pragma unroll 8
  for (int s = g; s < splits; s += kCombGroups) {
    const int64_t qi = int64_t(s) * Hq + i;
    const float m = ws_ml[2 * qi];
    const float w = m == -__builtin_inff() ? 0.0f : __expf(m - M);
    L = __builtin_fmaf(ws_ml[2 * qi + 1], w, L);
    O = __builtin_fmaf(ws_o[qi * kAttnD + c], w, O);
  }
  s_red[tid] = O;
  s_l[tid] = L;
  __syncthreads();
  if (g == 0) {
    float Ot = 0.0f, Lt = 0.0f;
#pragma unroll
    for (int k = 0; k < kCombGroups; ++k) {
      Ot += s_red[k * kCombChannels + tid];
      Lt += s_l[k * kCombChannels + tid];
    }
    out[int64_t(i) * kAttnD + c] = __builtin_bit_cast(uint16_t, (__bf16)(Ot / Lt));
    if (out32) out32[int64_t(i) * kAttnD + c] = Ot / Lt;     // the sparse reference's O_ref
    if (ml_out && c == 0) {                                   // and its softmax max and denominator
      ml_out[2 * i] = M;
      ml_out[2 * i + 1] = Lt;
    }
  }
}

template <bool SC, int FMT = 0>
static hipError_t launch_attn(int32_t T, int32_t H, int32_t Hq, const void* q, const ChainArgs& kc,
                              const ChainArgs& vc, const void* k_tail, const void* v_tail, int32_t tail_len,
                              float scale, void* out, float* out32, float* ml_out, float* scores, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  if (ws == nullptr || ws_bytes < attn_workspace_need(T, tail_len, H, Hq)) return hipErrorInvalidValue;
  const int32_t tiles = attn_tiles(T, tail_len);
  // Chains with packed tokens take the two-pass reader (the score-writing call only without a
  // tail, whose scores rows count the packed positions alone); FP4 chains without a tail and of
  // at most kSplitFp4Loops loops
  const bool two_pass = T > 0 && (!SC || tail_len == 0) &&
                        (FMT == 0 || (tail_len == 0 && kc.n_loops <= kSplitFp4Loops && vc.n_loops <= kSplitFp4Loops));
  const int32_t nw = two_pass ? kSplitAttnWaves : kAttnWaves;
  const int32_t wph = waves_per_head(tiles, H, nw);
  const int32_t splits = n_splits(tiles, H, nw);
  const int32_t G = Hq / H;
  float* ws_ml = static_cast<float*>(ws);
  float* ws_o = ws_ml + size_t(splits) * Hq * 2;
  const uint16_t* qp = static_cast<const uint16_t*>(q);
  const uint16_t* ktp = static_cast<const uint16_t*>(k_tail);
  const uint16_t* vtp = static_cast<const uint16_t*>(v_tail);
  int nl = kc.n_loops > vc.n_loops ? kc.n_loops : vc.n_loops;
  if (nl < 1) nl = 1;                              // no packed tokens: only the tail's tiles run
  const dim3 grid(static_cast<unsigned>(splits), static_cast<unsigned>(H));
  if (two_pass) {
    // INT4 chains: the scores of every position (packed, then the BF16 tail), then PV straight
    // from the V codes (the tail's V as stored)
    float* block_max = ws_o + size_t(splits) * Hq * kAttnD;
    float* sc = SC ? scores : block_max + size_t(splits) * Hq;
    const hipError_t e = launch_attn_split(FMT, T, H, Hq, q, kc, vc, k_tail, v_tail, tail_len, scale, wph, splits, sc,
                                           block_max, ws_ml, ws_o, stream);
    if (e != hipSuccess) return e;
  } else {
#define FLK_A(NLV)                                                                                          \
  case NLV:                                                                                                 \
    hipLaunchKernelGGL((attn_wave_kernel<NLV, SC, FMT>), grid, dim3(kAThreads), 0, stream, kc, vc, T, H, G, qp, \
                       ktp, vtp, tail_len, scale, wph, ws_ml, ws_o, scores);                                \
    break;
    switch (nl) {
      FLK_A(1) FLK_A(2) FLK_A(3) FLK_A(4) FLK_A(5) FLK_A(6) FLK_A(7) FLK_A(8)
      default: return hipErrorInvalidValue;
    }
#undef FLK_A
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(attn_combine_kernel, dim3(Hq, kAttnD / kCombChannels), dim3(kCombThreads), 0, stream, splits, Hq, ws_ml,
                     ws_o, static_cast<uint16_t*>(out), out32, ml_out);
  return hipGetLastError();
}

hipError_t launch_decode_attn(int32_t T, int32_t H, int32_t D, int32_t Hq, const void* q,
                              const ChainArgs& kc, const ChainArgs& vc, const void* k_tail,
                              const void* v_tail, int32_t tail_len, float scale, void* out,
                              void* ws, size_t ws_bytes, hipStream_t stream) {
  (void)D;
  return launch_attn<false>(T, H, Hq, q, kc, vc, k_tail, v_tail, tail_len, scale, out, nullptr, nullptr, nullptr,
                            ws, ws_bytes, stream);
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];    // device address of `scratch` per device, found once

// The current device's copy of `scratch`, looked up on the first call on that device.
hipError_t scratch_address(void** p) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *p = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

hipError_t launch_decode_attn_noalloc(int32_t T, int32_t H, int32_t D, int32_t Hq, const void* q, const ChainArgs& kc,
                                      const ChainArgs& vc, float scale, void* out, hipStream_t stream) {
  if (attn_workspace_need(T, 0, H, Hq) > size_t(FLK_NOALLOC_SCRATCH_BYTES)) return hipErrorInvalidValue;
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return e;
  // every partial the combine reads is written by the attention kernel first: nothing to clear
  return launch_decode_attn(T, H, D, Hq, q, kc, vc, nullptr, nullptr, 0, scale, out, ws,
                            size_t(FLK_NOALLOC_SCRATCH_BYTES), stream);
}

hipError_t launch_decode_attn_fmt(int fmt, int32_t T, int32_t H, int32_t Hq, const void* q, const ChainArgs& kc,
                                  const ChainArgs& vc, float scale, void* out, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  switch (fmt) {
    case 0:
      return launch_attn<false, 0>(T, H, Hq, q, kc, vc, nullptr, nullptr, 0, scale, out, nullptr, nullptr, nullptr, ws,
                                   ws_bytes, stream);
    case 1:
      return launch_attn<false, 1>(T, H, Hq, q, kc, vc, nullptr, nullptr, 0, scale, out, nullptr, nullptr, nullptr, ws,
                                   ws_bytes, stream);
    case 2:
      return launch_attn<false, 2>(T, H, Hq, q, kc, vc, nullptr, nullptr, 0, scale, out, nullptr, nullptr, nullptr, ws,
                                   ws_bytes, stream);
    case 3:
      return launch_attn<false, 3>(T, H, Hq, q, kc, vc, nullptr, nullptr, 0, scale, out, nullptr, nullptr, nullptr, ws,
                                   ws_bytes, stream);
    case 4:
      return launch_attn<false, 4>(T, H, Hq, q, kc, vc, nullptr, nullptr, 0, scale, out, nullptr, nullptr, nullptr, ws,
                                   ws_bytes, stream);
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_reference(int fmt, int32_t T, int32_t H, int32_t Hq, const void* q, const ChainArgs& kc,
                                 const ChainArgs& vc, float scale, void* out, float* o_ref, float* ml,
                                 float* scores, void* ws, size_t ws_bytes, hipStream_t stream) {
#define FLK_R(F)                                                                                                  \
  case F:                                                                                                         \
    return launch_attn<true, F>(T, H, Hq, q, kc, vc, nullptr, nullptr, 0, scale, out, o_ref, ml, scores, ws,      \
                                ws_bytes, stream);
  switch (fmt) {
    FLK_R(0) FLK_R(1) FLK_R(2) FLK_R(3) FLK_R(4)
    default: return hipErrorInvalidValue;
  }
#undef FLK_R
}

}  // namespace flk
