// Predicated chunk copy through the LDS copy pipeline, for chunks of W = 16
// bytes and, with the same schedule, W = 8 and 4 bytes.
//
// Semantics ("Asynchronous Copies", section "A Global-to-Shared Copy", the
// paragraph on the copy's operands): a false pred skips the copy and leaves
// the destination unchanged; src_size copies a byte prefix and zero-fills the
// rest; ignore_src zero-fills the whole chunk. The copy itself is skipped
// whenever it would bring no byte that survives (pred false, ignore_src set,
// or src_size 0): those lanes get the first out-of-range offset (the end of
// the workgroup's run), so the load moves nothing, while the instruction still
// issues and the wait counts hold.
//
// One lane owns one chunk of a 256-chunk tile. Per tile, each wave issues
//   three 1-byte LDS-DMA loads (pred, src_size, ignore_src of its 64 chunks)
//   one 16-byte LDS-DMA load of its 64 chunks (W = 16 with a 16-byte-aligned
//   source), or else W/4 4-byte loads covering the wave's 64 * W bytes, word
//   after word, so every chunk lands contiguously at LDS byte tid * W
// and on consumption reads its chunk and the three bytes back from LDS,
// zeroes the bytes past the prefix and stores W bytes (one 16-byte store or
// W/4 words), with
// the store's offset out of range when pred is false, so the destination is
// never written there. Everything a lane reads from LDS was loaded by its own
// wave, so the per-wave vmcnt wait is the whole synchronization; no workgroup
// barrier is needed.
//
// Schedule (S data slots, 2S-1 metadata slots): a tile's metadata is loaded
// S-1 iterations before its data, in the same issue group as the data of an
// earlier tile. Because loads retire in order, the wait for tile t's data
// also guarantees that the metadata of tile t+S-1, needed to mask that tile's
// data load in the same iteration, has landed.
//   prologue: meta 0 .. S-2; wait for all; then groups g = 0 .. S-2:
//             {meta g+S-1, data g}
//   iteration t: wait (data t landed)
//                issue group {meta t+2S-2, data t+S-1 masked by meta t+S-1}
//                consume t (meta t, data t)
#include "tp_engine.hpp"
#include "tp_internal.hpp"

namespace tp {
namespace dev {

template <int S, int W, bool LX4, bool SX4>
__global__ void __launch_bounds__(256) chunk_copy_kernel(ChunkParams p)
{
    static_assert(W == 16 || ((W == 8 || W == 4) && !LX4 && !SX4), "narrow chunks move as words");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr int R = chunk_meta_slots(S);
    constexpr int LD = chunk_loads_per_tile(LX4, W);
    constexpr int ST = chunk_stores_per_tile(SX4, W);
    constexpr int WPC = W / 4;                        // words per chunk
    constexpr uint32_t kData = chunk_data_slot_bytes(W);   // 256 chunks per data slot
    constexpr uint32_t kMeta = kChunkMetaSlotBytes;   // 3 KiB per metadata slot

    const uint32_t tid = threadIdx.x;
    const uint32_t wave_first = uniform(tid & ~63u);
    const uint32_t lane = tid - wave_first;
    const int64_t first = (int64_t)blockIdx.x * p.tiles_per_block * kChunkTile;
    const int64_t rem = p.n_chunks - first;
    const int64_t run = (int64_t)p.tiles_per_block * kChunkTile;
    const uint32_t span = (uint32_t)(rem < run ? rem : run);   // chunks of this workgroup
    const int cnt = (int)((span + kChunkTile - 1) / kChunkTile);
    const bool has_pred = p.flags & kHasPred;
    const bool has_size = p.flags & kHasSize;
    const bool has_ign = p.flags & kHasIgnore;

    const uint32_t run_end = span * W;            // first out-of-range byte of src/dst
    const BufferRes rsrc = make_buffer_res(p.src + W * first, run_end);
    const BufferRes rdst = make_buffer_res(p.dst + W * first, run_end);
    // An absent metadata array still gets its loads issued (so counts stay
    // fixed); they read the run's own source bytes, and those LDS bytes are
    // ignored.
    const uint8_t *src_run = p.src + W * first;
    const BufferRes rpred = make_buffer_res(has_pred ? p.pred + first : src_run, span);
    const BufferRes rsize = make_buffer_res(has_size ? p.src_size + first : src_run, span);
    const BufferRes rign = make_buffer_res(has_ign ? p.ignore_src + first : src_run, span);

    const uint32_t base = uniform(lds_offset(lds));
    const uint32_t data_ring = 0;                 // offsets from `lds`
    const uint32_t meta_ring = S * kData;
    // metadata slot layout: [wave][array][64 lanes x 4 bytes]
    const uint32_t meta_wave = wave_first * 12;   // = (wave_first / 64) * 768

    auto issue_meta = [&](uint32_t j, uint32_t mslot) TP_INLINE {
        const uint32_t voff = j * kChunkTile + tid;
        const uint32_t m0 = base + meta_ring + mslot * kMeta + meta_wave;
        dma_u8(rpred, voff, uniform(m0));
        dma_u8(rsize, voff, uniform(m0 + 256));
        dma_u8(rign, voff, uniform(m0 + 512));
    };

    // Effective byte count of the lane's chunk (0..W) and whether it is stored.
    struct Meta {
        uint32_t keep;
        bool store;
    };
    auto read_meta = [&](uint32_t mslot) TP_INLINE {
        const uint8_t *m = lds + meta_ring + mslot * kMeta + meta_wave + lane * 4;
        const bool pr = has_pred ? m[0] != 0 : true;
        const bool ig = has_ign ? m[512] != 0 : false;
        uint32_t s = has_size ? m[256] : (uint32_t)W;
        s = s > (uint32_t)W ? (uint32_t)W : s;
        return Meta{ig ? 0u : s, pr};
    };

    auto issue_data = [&](uint32_t j, uint32_t dslot, uint32_t mslot) TP_INLINE {
        const uint32_t slot = base + data_ring + dslot * kData;
        if constexpr (LX4) {
            const Meta m = read_meta(mslot);
            const bool needed = m.store && m.keep != 0;
            dma_b128(rsrc, needed ? j * kData + tid * 16 : run_end, uniform(slot + wave_first * 16));
        } else {
            static_for<0, WPC>([&](auto q) TP_INLINE {
                const uint32_t w0 = wave_first * WPC + q * 64;   // first word of this load
                dma_b32(rsrc, j * kData + (w0 + lane) * 4, uniform(slot + w0 * 4));
            });
        }
    };

    auto consume = [&](uint32_t j, uint32_t dslot, uint32_t mslot) TP_INLINE {
        const Meta m = read_meta(mslot);
        u32x4 v;
        if constexpr (W == 16) {
            v = *reinterpret_cast<const u32x4 *>(lds + data_ring + dslot * kData + tid * 16);
        } else {
            static_for<0, WPC>([&](auto w) TP_INLINE {
                v[(int)w] = *reinterpret_cast<const uint32_t *>(lds + data_ring + dslot * kData + tid * W + w * 4);
            });
        }
        // keep bytes [0, keep): word w keeps min(max(keep - 4w, 0), 4) bytes
#pragma unroll
        for (int w = 0; w < WPC; ++w) {
            const int kb = (int)m.keep - 4 * w;
            const uint32_t mask = kb >= 4 ? 0xFFFFFFFFu : kb <= 0 ? 0u : ((1u << (8 * kb)) - 1u);
            v[w] &= mask;
        }
        const uint32_t off = j * kData + tid * W;
        if constexpr (SX4) {
            store_b128(rdst, m.store ? off : run_end, v);
        } else {
            static_for<0, WPC>([&](auto w) TP_INLINE { store_b32(rdst, m.store ? off + w * 4 : run_end, v[(int)w]); });
        }
    };

    if constexpr (S == 1) {
        for (int t = 0; t < cnt; ++t) {
            issue_meta(t, 0);
            vm_wait<0>();
            issue_data(t, 0, 0);
            vm_wait<0>();
            consume(t, 0, 0);
        }
    } else {
        static_for<0, S - 1>([&](auto m) TP_INLINE { issue_meta(m, m); });
        vm_wait<0>();
        static_for<0, S - 1>([&](auto g) TP_INLINE {
            issue_meta(g + S - 1, g + S - 1);
            issue_data(g, g, g);
        });
        bool stop = false;
        static_for<0, S - 1>([&](auto T) TP_INLINE {
            if (!stop) {
                if ((int)T >= cnt) {
                    stop = true;
                } else {
                    vm_wait<stage_wait_count(S, LD, ST, T)>();
                    issue_meta(T + 2 * S - 2, (T + 2 * S - 2) % R);
                    issue_data(T + S - 1, (T + S - 1) % S, (T + S - 1) % R);
                    consume(T, T % S, T % R);
                }
            }
        });
        uint32_t dcur = (S - 1) % S;   // data slot of tile t
        uint32_t mcur = (S - 1) % R;   // metadata slot of tile t
        for (int t = S - 1; t < cnt; ++t) {
            const uint32_t dnxt = dcur == 0 ? S - 1 : dcur - 1;              // (t + S - 1) mod S
            const uint32_t mnxt = mcur + S - 1 >= R ? mcur + S - 1 - R : mcur + S - 1;  // (t + S - 1) mod R
            const uint32_t mfar = mcur == 0 ? R - 1 : mcur - 1;              // (t + 2S - 2) mod R
            vm_wait<stage_wait_count(S, LD, ST, S - 1)>();
            issue_meta(t + 2 * S - 2, mfar);
            issue_data(t + S - 1, dnxt, mnxt);
            consume(t, dcur, mcur);
            dcur = dcur + 1 == S ? 0 : dcur + 1;
            mcur = mcur + 1 == R ? 0 : mcur + 1;
        }
    }
    // No copy into LDS may still be in flight when the workgroup's LDS is freed.
    vm_wait<0>();
}

}  // namespace dev

int launch_chunk_copy(const tp_plan &plan, const ChunkParams &p, void *stream)
{
    using Fn = void (*)(ChunkParams);
    // per stage count: the four 16-byte-chunk paths, then 8- and 4-byte chunks (words only)
#define TP_CHUNK_ROW(S)                                                                        \
    &dev::chunk_copy_kernel<S, 16, true, true>, &dev::chunk_copy_kernel<S, 16, false, true>,   \
        &dev::chunk_copy_kernel<S, 16, true, false>, &dev::chunk_copy_kernel<S, 16, false, false>, \
        &dev::chunk_copy_kernel<S, 8, false, false>, &dev::chunk_copy_kernel<S, 4, false, false>
    static constexpr Fn table[kMaxStages * 6] = {TP_CHUNK_ROW(1), TP_CHUNK_ROW(2), TP_CHUNK_ROW(3),
                                                 TP_CHUNK_ROW(4), TP_CHUNK_ROW(5), TP_CHUNK_ROW(6),
                                                 TP_CHUNK_ROW(7), TP_CHUNK_ROW(8)};
#undef TP_CHUNK_ROW
    const int col = plan.chunk_bytes == 16 ? plan.path : plan.chunk_bytes == 8 ? 4 : 5;
    const Fn fn = table[(plan.stages - 1) * 6 + col];
    if (plan.lds_bytes > 65536) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 plan.lds_bytes);
        if (e != hipSuccess)
            return (int)e;
    }
    ChunkParams args = p;
    void *kargs[] = {&args};
    return (int)hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3((uint32_t)plan.grid),
                                dim3((uint32_t)plan.threads), kargs, (size_t)plan.lds_bytes,
                                (hipStream_t)stream);
}

}  // namespace tp
