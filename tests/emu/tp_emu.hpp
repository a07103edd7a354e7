// CPU emulator of the library's kernel bodies (test infrastructure): the
// emulated engine and the scheduler.
//
// The kernel bodies of libtilepipe are templates on an engine type. The
// library instantiates them with the gfx950 engine; tp_emu_*.cpp instantiate
// the very same source with the emulated engine below and run a planned launch
// on the host, one workgroup after another (one launch at a time per process:
// the scheduler's state is global). Every lane is a fiber; the lanes of a
// wave run in lock-step from one engine call to the next, and each engine call
// is executed once for the whole wave, as the hardware executes one
// instruction for 64 lanes. At every call the emulator checks what a GPU run
// would otherwise only show as a fault, a hang or a wrong value now and then:
//
//   memory     an access whose offset passes the buffer's range check must lie
//              inside a buffer the caller registered (reads) or registered as
//              writable (writes). Lanes failing the range check move nothing;
//              a direct-to-LDS load writes zeros to their LDS slot.
//   LDS        every LDS access stays inside the workgroup's allocation; no
//              byte is read that no load of this workgroup wrote.
//   waits      a wave's vector-memory operations retire in issue order, and
//              only at a wait: s_waitcnt vmcnt(K) retires the oldest until at
//              most K are outstanding (and issue stalls, retiring the oldest,
//              when 63 are outstanding). Reading LDS bytes whose load has not
//              retired is an error: the hardware could return the slot's old
//              contents.
//   sharing    LDS bytes written by one wave and read by another (or read by
//              one wave and then overwritten by another's load) need a barrier
//              in between, with the load retired before it.
//   the end    no direct-to-LDS load may still be in flight when a wave ends.
//   lock-step  every lane of a wave reaches the same engine call; the values
//              given to readfirstlane and M0 are the same on every lane.
//
// Two landing policies bracket the hardware's timing: "late" moves a load's
// bytes at its retirement (the latest the hardware may), "early" at its issue.
// The waves of a workgroup are interleaved in a seeded random order.
#pragma once

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
#include <ucontext.h>

#include <algorithm>
#include <deque>
#include <functional>
#include <memory>
#include <random>
#include <stdexcept>
#include <string>
#include <type_traits>
#include <vector>

#include "tp_engine.hpp"
#include "tp_internal.hpp"

namespace emu {

using tp::dev::u32x4;

struct Region {
    uint64_t lo, hi;
    int writable;
};

struct Options {
    int policy;          // 0: loads land at retirement, 1: at issue
    int wait_bias;       // added to every wait count (a planted mistake when > 0)
    uint64_t seed;       // order in which ready waves are stepped
    uint32_t lds_base;   // LDS address of the workgroup's dynamic LDS
    const Region *regions;
    int n_regions;
    const int64_t *blocks;   // workgroups to run (all when null)
    int n_blocks;
    int oor_fill;        // what an out-of-range lane's load leaves in its LDS slot:
                         // 0 zeros (measured on the MI355X), 1 random bytes (the
                         // kernels must not depend on it)
    int drop_barriers;   // a planted mistake: workgroup barriers do nothing
};

struct Fail : std::runtime_error {
    using std::runtime_error::runtime_error;
};

[[noreturn]] inline void fail(const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    throw Fail(buf);
}

struct Res {
    uint64_t base;
    uint32_t num_records;
};

enum Kind { K_NONE, K_UNIFORM, K_LDS_LOAD, K_DMA, K_STORE, K_WAIT, K_BARRIER, K_DONE, K_LDS_STORE,
            K_LOAD, K_ALL };

inline const char *kind_name(int k)
{
    static const char *n[] = {"none", "readfirstlane", "LDS read", "LDS-DMA load", "store",
                              "vmcnt wait", "barrier", "end", "LDS write", "register load",
                              "ballot"};
    return n[k];
}

struct Request {
    int kind = K_NONE;
    uint32_t a = 0, b = 0;   // UNIFORM: a = value; LDS_LOAD, LDS_STORE: a = offset, b = size;
                             // DMA: a = voff, b = m0; STORE, LOAD: a = voff; WAIT: a = K;
                             // ALL: a = the lane's predicate
    int width = 0;           // DMA/STORE: 16, 8, 4 or 1 bytes; LOAD: 8 or 4
    Res res{};
    uint8_t data[16];        // STORE and LDS_STORE data, LDS_LOAD result
    uint32_t result = 0;     // UNIFORM, ALL and 4-byte LOAD result
    uint64_t wide = 0;       // 8-byte LOAD result
};

struct Lane {
    ucontext_t ctx;
    uint32_t tid = 0;
    bool done = false;
    Request req;
};

struct Xfer {
    uint32_t lds;            // LDS index (from lds[0]) of the lane's slot
    uint32_t slot;           // bytes written to LDS
    uint64_t addr[16];       // global address of each byte, or 0 for zero-fill
    int nbytes;              // bytes taken from memory (1, 4 or 16)
};

struct VmOp {
    bool load;
    int64_t id;
    std::vector<Xfer> x;
};

struct Shadow {
    int64_t pending = -1;    // id of the in-flight load that writes this byte
    int16_t writer = -1;     // wave of the last load or LDS write that wrote it (-1: never)
    int64_t write_epoch = 0; // barrier epoch in which that load retired (or the write ran)
    uint32_t readers = 0;    // waves that read it in epoch read_epoch (bit mask)
    int64_t read_epoch = -1;
};

struct Wave {
    int id;
    std::vector<Lane *> lanes;
    std::deque<VmOp> vm;
    bool at_barrier = false;
    bool done = false;
};

class Emulator;
inline Emulator *g_emu = nullptr;
inline Lane *g_lane = nullptr;

class Emulator {
  public:
    Emulator(const Options &o, uint32_t threads, uint32_t lds_bytes, uint32_t grid)
        : opt(o), nthreads(threads), lds_bytes(lds_bytes), grid(grid), rng(o.seed)
    {
        if (threads == 0 || threads > 1024)
            fail("workgroup of %u lanes", threads);
        if ((uint64_t)o.lds_base + lds_bytes > 160u * 1024u)
            fail("LDS allocation of %u bytes at %u exceeds 160 KiB", lds_bytes, o.lds_base);
        for (uint32_t t = 0; t < threads; ++t)
            stacks.emplace_back(new char[kStack]);
    }

    template <class Body>
    void run(Body body)
    {
        std::vector<int64_t> blocks;
        if (opt.blocks)
            blocks.assign(opt.blocks, opt.blocks + opt.n_blocks);
        else
            for (uint32_t b = 0; b < grid; ++b)
                blocks.push_back(b);
        body_ = body;
        for (int64_t b : blocks) {
            if (b < 0 || b >= (int64_t)grid)
                fail("workgroup %lld is outside the grid of %u", (long long)b, grid);
            run_block((uint32_t)b);
        }
    }

    // ----------------------------------------------------------- engine side
    uint32_t block_id() const { return block; }
    uint32_t grid_size() const { return grid; }
    uint32_t threads() const { return nthreads; }
    uint32_t lds_base() const { return opt.lds_base; }
    uint8_t *lds_data() { return lds.data(); }

    // Post the calling lane's request and give control back to the scheduler.
    void post(const Request &r)
    {
        g_lane->req = r;
        swapcontext(&g_lane->ctx, &sched);
    }

  private:
    Options opt;
    uint32_t nthreads, lds_bytes, grid;
    std::mt19937_64 rng;
    std::mt19937 oor_rng{12345};
    std::function<void()> body_;
    uint32_t block = 0;
    ucontext_t sched;
    std::vector<uint8_t> lds;
    std::vector<Shadow> shadow;
    std::vector<Wave> waves;
    std::vector<Lane> lanes;
    static constexpr size_t kStack = 128 * 1024;
    std::vector<std::unique_ptr<char[]>> stacks;
    int64_t epoch = 0;
    int64_t next_op = 0;

    static void trampoline()
    {
        g_emu->body_();
        g_emu->post(Request{K_DONE});
        // never resumed after K_DONE
    }

    const Region *region_of(uint64_t lo, uint64_t n) const
    {
        for (int i = 0; i < opt.n_regions; ++i)
            if (lo >= opt.regions[i].lo && lo + n <= opt.regions[i].hi)
                return &opt.regions[i];
        return nullptr;
    }

    void run_block(uint32_t b)
    {
        block = b;
        epoch = 0;
        lds.assign(lds_bytes, 0);
        std::mt19937 fill((uint32_t)(opt.seed * 2654435761u + b));
        for (auto &v : lds)
            v = (uint8_t)fill();   // LDS holds whatever an earlier workgroup left
        shadow.assign(lds_bytes, Shadow{});
        const uint32_t nw = (nthreads + 63) / 64;
        lanes.assign(nthreads, Lane{});
        waves.assign(nw, Wave{});
        for (uint32_t w = 0; w < nw; ++w)
            waves[w].id = (int)w;
        for (uint32_t t = 0; t < nthreads; ++t) {
            Lane &l = lanes[t];
            l.tid = t;
            getcontext(&l.ctx);
            l.ctx.uc_stack.ss_sp = stacks[t].get();
            l.ctx.uc_stack.ss_size = kStack;
            l.ctx.uc_link = nullptr;
            makecontext(&l.ctx, (void (*)())trampoline, 0);
            waves[t / 64].lanes.push_back(&l);
        }
        for (;;) {
            std::vector<int> ready;
            int live = 0;
            for (auto &w : waves) {
                if (w.done)
                    continue;
                ++live;
                if (!w.at_barrier)
                    ready.push_back(w.id);
            }
            if (live == 0)
                break;
            if (ready.empty()) {       // every live wave is at the barrier
                ++epoch;
                for (auto &w : waves)
                    w.at_barrier = false;
                continue;
            }
            step(waves[ready[rng() % ready.size()]]);
        }
    }

    // Run every lane of the wave to its next engine call, then execute it.
    void step(Wave &w)
    {
        for (Lane *l : w.lanes) {
            g_lane = l;
            swapcontext(&sched, &l->ctx);
        }
        g_lane = nullptr;
        const int kind = w.lanes[0]->req.kind;
        for (Lane *l : w.lanes)
            if (l->req.kind != kind)
                fail("workgroup %u wave %d: lane %u reached a %s while lane %u reached a %s "
                     "(lanes of a wave left lock-step)", block, w.id, w.lanes[0]->tid,
                     kind_name(kind), l->tid, kind_name(l->req.kind));
        switch (kind) {
        case K_UNIFORM: {
            const uint32_t v = w.lanes[0]->req.a;
            for (Lane *l : w.lanes) {
                if (l->req.a != v)
                    fail("workgroup %u wave %d: readfirstlane of a value that differs between "
                         "lanes (%u on lane %u, %u on lane %u)", block, w.id, v, w.lanes[0]->tid,
                         l->req.a, l->tid);
                l->req.result = v;
            }
            break;
        }
        case K_LDS_LOAD: lds_read(w); break;
        case K_LDS_STORE: lds_write(w); break;
        case K_LOAD: reg_load(w); break;
        case K_ALL: {
            uint32_t all = 1;
            for (Lane *l : w.lanes)
                all &= l->req.a != 0;
            for (Lane *l : w.lanes)
                l->req.result = all;
            break;
        }
        case K_DMA: dma(w); break;
        case K_STORE: store(w); break;
        case K_WAIT: {
            const uint32_t k = w.lanes[0]->req.a;
            for (Lane *l : w.lanes)
                if (l->req.a != k)
                    fail("wave %d: lanes wait for different counts", w.id);
            const int kk = std::min<int>((int)k + opt.wait_bias, tp::kVmcntMax);
            while ((int)w.vm.size() > kk)
                retire(w);
            break;
        }
        case K_BARRIER: w.at_barrier = !opt.drop_barriers; break;
        case K_DONE:
            for (const VmOp &op : w.vm)
                if (op.load)
                    fail("workgroup %u wave %d ended with a direct-to-LDS load in flight "
                         "(the workgroup's LDS may be handed on before it lands)", block, w.id);
            w.vm.clear();
            w.done = true;
            break;
        default: fail("unknown request");
        }
    }

    void lds_read(Wave &w)
    {
        for (Lane *l : w.lanes) {
            const uint32_t off = l->req.a, n = l->req.b;
            if ((uint64_t)off + n > lds_bytes)
                fail("workgroup %u wave %d lane %u: LDS read of %u bytes at %u, outside the "
                     "%u-byte allocation", block, w.id, l->tid, n, off, lds_bytes);
            for (uint32_t i = 0; i < n; ++i) {
                Shadow &s = shadow[off + i];
                if (s.pending >= 0)
                    fail("workgroup %u wave %d lane %u: LDS byte %u read while the load that "
                         "writes it is still in flight (a wait count too small)", block, w.id,
                         l->tid, off + i);
                if (s.writer < 0)
                    fail("workgroup %u wave %d lane %u: LDS byte %u read, but no load of this "
                         "workgroup wrote it", block, w.id, l->tid, off + i);
                if (s.writer != w.id && s.write_epoch >= epoch)
                    fail("workgroup %u wave %d lane %u: LDS byte %u was written by wave %d with "
                         "no barrier between its load's retirement and this read", block, w.id,
                         l->tid, off + i, s.writer);
                if (s.read_epoch != epoch) {
                    s.read_epoch = epoch;
                    s.readers = 0;
                }
                s.readers |= 1u << w.id;
            }
            memcpy(l->req.data, lds.data() + off, n);
        }
    }

    // A wave's own LDS write: it lands at once (LDS operations of a wave run in
    // order). The bytes must not be the target of a load still in flight, nor
    // have been read or written by another wave since the last barrier.
    void lds_write(Wave &w)
    {
        for (Lane *l : w.lanes) {
            const uint32_t off = l->req.a, n = l->req.b;
            if ((uint64_t)off + n > lds_bytes)
                fail("workgroup %u wave %d lane %u: LDS write of %u bytes at %u, outside the "
                     "%u-byte allocation", block, w.id, l->tid, n, off, lds_bytes);
            for (uint32_t i = 0; i < n; ++i) {
                Shadow &s = shadow[off + i];
                if (s.pending >= 0)
                    fail("workgroup %u wave %d lane %u: LDS write to byte %u while a load that "
                         "writes it is still in flight", block, w.id, l->tid, off + i);
                if (s.read_epoch == epoch && (s.readers & ~(1u << w.id)))
                    fail("workgroup %u wave %d lane %u: LDS write to byte %u, which another "
                         "wave read with no barrier in between", block, w.id, l->tid, off + i);
                if (s.writer >= 0 && s.writer != w.id && s.write_epoch >= epoch)
                    fail("workgroup %u wave %d lane %u: LDS write to byte %u, which wave %d "
                         "wrote with no barrier in between", block, w.id, l->tid, off + i,
                         s.writer);
                s.writer = (int16_t)w.id;
                s.write_epoch = epoch;
            }
            memcpy(lds.data() + off, l->req.data, n);
        }
    }

    void dma(Wave &w)
    {
        const int width = w.lanes[0]->req.width;
        const uint32_t m0 = w.lanes[0]->req.b;
        const uint32_t slot = width == 16 ? 16 : 4;
        if (w.vm.size() >= (size_t)tp::kVmcntMax)
            retire(w);   // issue stalls until one retires
        VmOp op{true, next_op++, {}};
        for (size_t li = 0; li < w.lanes.size(); ++li) {
            Lane *l = w.lanes[li];
            if (l->req.b != m0 || l->req.width != width)
                fail("workgroup %u wave %d: M0 differs between lanes of one load", block, w.id);
            const uint64_t a = (uint64_t)m0 + li * slot;
            if (a < opt.lds_base || a + slot > (uint64_t)opt.lds_base + lds_bytes)
                fail("workgroup %u wave %d lane %u: LDS-DMA slot at LDS address %llu, outside "
                     "the allocation [%u, %u)", block, w.id, l->tid, (unsigned long long)a,
                     opt.lds_base, opt.lds_base + lds_bytes);
            Xfer x;
            x.lds = (uint32_t)(a - opt.lds_base);
            x.slot = slot;
            x.nbytes = width;
            const Res &r = l->req.res;
            const uint32_t voff = l->req.a;
            for (int i = 0; i < 16; ++i)
                x.addr[i] = 0;
            // the range check, per dword (per byte for the 1-byte load)
            const int unit = width == 1 ? 1 : 4;
            for (int k = 0; k < width; k += unit) {
                const uint64_t o = (uint64_t)voff + k;
                if (o + unit > r.num_records)
                    continue;
                const uint64_t g = r.base + o;
                if (!region_of(g, unit))
                    fail("workgroup %u wave %d lane %u: load of %d bytes at offset %llu of a "
                         "buffer at %#llx (num_records %u) reads outside every buffer of the "
                         "call", block, w.id, l->tid, unit, (unsigned long long)o,
                         (unsigned long long)r.base, r.num_records);
                for (int i = 0; i < unit; ++i)
                    x.addr[k + i] = g + i;
            }
            for (uint32_t i = 0; i < slot; ++i) {
                Shadow &s = shadow[x.lds + i];
                if (s.pending >= 0)
                    fail("workgroup %u wave %d lane %u: LDS-DMA into byte %u, which an earlier "
                         "load still in flight also writes", block, w.id, l->tid, x.lds + i);
                if (s.read_epoch == epoch && (s.readers & ~(1u << w.id)))
                    fail("workgroup %u wave %d lane %u: LDS-DMA into byte %u, which another "
                         "wave read with no barrier in between", block, w.id, l->tid, x.lds + i);
                if (s.writer >= 0 && s.writer != w.id && s.write_epoch >= epoch)
                    fail("workgroup %u wave %d lane %u: LDS-DMA into byte %u, which wave %d "
                         "wrote with no barrier in between", block, w.id, l->tid, x.lds + i,
                         s.writer);
                s.pending = op.id;
            }
            op.x.push_back(x);
        }
        if (opt.policy == 1)
            land(op);
        w.vm.push_back(std::move(op));
    }

    void land(const VmOp &op)
    {
        for (const Xfer &x : op.x) {
            uint8_t v[16] = {0};
            for (int i = 0; i < x.nbytes; ++i)
                v[i] = x.addr[i] ? *reinterpret_cast<const uint8_t *>(x.addr[i])
                                 : opt.oor_fill ? (uint8_t)oor_rng() : 0;
            if (x.nbytes == 1 && !x.addr[0] && opt.oor_fill)
                for (uint32_t i = 1; i < x.slot; ++i)
                    v[i] = (uint8_t)oor_rng();
            memcpy(lds.data() + x.lds, v, x.slot);   // a 1-byte load fills a dword, zero-extended
        }
    }

    void retire(Wave &w)
    {
        VmOp op = std::move(w.vm.front());
        w.vm.pop_front();
        if (!op.load)
            return;
        if (opt.policy == 0)
            land(op);
        for (const Xfer &x : op.x)
            for (uint32_t i = 0; i < x.slot; ++i) {
                Shadow &s = shadow[x.lds + i];
                s.pending = -1;
                s.writer = (int16_t)w.id;
                s.write_epoch = epoch;
            }
    }

    // A 4-byte load into a register whose block ends with vmcnt(0): every
    // earlier operation of the wave retires first, then each lane reads (0
    // when its offset fails the range check).
    void reg_load(Wave &w)
    {
        while (!w.vm.empty())
            retire(w);
        for (Lane *l : w.lanes) {
            const Res &r = l->req.res;
            const uint64_t o = l->req.a;
            const int width = l->req.width == 8 ? 8 : 4;
            uint64_t v = 0;
            if (o + width <= r.num_records) {
                const uint64_t g = r.base + o;
                if (!region_of(g, width))
                    fail("workgroup %u wave %d lane %u: load of %d bytes at offset %llu of a "
                         "buffer at %#llx (num_records %u) reads outside every buffer of the "
                         "call", block, w.id, l->tid, width, (unsigned long long)o,
                         (unsigned long long)r.base, r.num_records);
                memcpy(&v, reinterpret_cast<const void *>(g), width);
            }
            l->req.result = (uint32_t)v;
            l->req.wide = v;
        }
    }

    void store(Wave &w)
    {
        const int width = w.lanes[0]->req.width;
        if (w.vm.size() >= (size_t)tp::kVmcntMax)
            retire(w);
        for (Lane *l : w.lanes) {
            const Res &r = l->req.res;
            for (int k = 0; k < width; k += 4) {
                const uint64_t o = (uint64_t)l->req.a + k;
                if (o + 4 > r.num_records)
                    continue;   // dropped by the range check
                const uint64_t g = r.base + o;
                const Region *reg = region_of(g, 4);
                if (!reg || !reg->writable)
                    fail("workgroup %u wave %d lane %u: store of 4 bytes at offset %llu of a "
                         "buffer at %#llx (num_records %u) writes outside every writable buffer "
                         "of the call", block, w.id, l->tid, (unsigned long long)o,
                         (unsigned long long)r.base, r.num_records);
                memcpy(reinterpret_cast<void *>(g), l->req.data + k, 4);
            }
        }
        w.vm.push_back(VmOp{false, next_op++, {}});
    }
};

// The engine the kernel bodies are instantiated with on the host.
struct EmuEngine {
    uint32_t tid() const { return g_lane->tid; }
    uint32_t nthreads() const { return g_emu->threads(); }
    uint32_t block() const { return g_emu->block_id(); }
    uint32_t blocks() const { return g_emu->grid_size(); }
    uint32_t uniform(uint32_t v) const
    {
        Request r;
        r.kind = K_UNIFORM;
        r.a = v;
        g_emu->post(r);
        return g_lane->req.result;
    }
    uint32_t lds_base() const { return g_emu->lds_base(); }
    template <class T>
    T lds_load(uint32_t off) const
    {
        Request r;
        r.kind = K_LDS_LOAD;
        r.a = off;
        r.b = sizeof(T);
        g_emu->post(r);
        T v;
        memcpy(&v, g_lane->req.data, sizeof(T));
        return v;
    }
    template <class T>
    void lds_store(uint32_t off, T v) const
    {
        static_assert(sizeof(T) <= 16, "LDS writes of at most 16 bytes");
        Request r;
        r.kind = K_LDS_STORE;
        r.a = off;
        r.b = sizeof(T);
        memcpy(r.data, &v, sizeof(T));
        g_emu->post(r);
    }
    Res res(const void *base, uint32_t num_records) const
    {
        // the descriptor is built from readfirstlane values
        const uint64_t a = reinterpret_cast<uint64_t>(base);
        const uint32_t lo = uniform((uint32_t)a), hi = uniform((uint32_t)(a >> 32) & 0xFFFFu);
        return Res{((uint64_t)hi << 32) | lo, uniform(num_records)};
    }
    void dma(const Res &r, uint32_t voff, uint32_t m0, int width) const
    {
        Request q;
        q.kind = K_DMA;
        q.a = voff;
        q.b = m0;
        q.width = width;
        q.res = r;
        g_emu->post(q);
    }
    void dma_b128(const Res &r, uint32_t voff, uint32_t m0) const { dma(r, voff, m0, 16); }
    void dma_b32(const Res &r, uint32_t voff, uint32_t m0) const { dma(r, voff, m0, 4); }
    void dma_u8(const Res &r, uint32_t voff, uint32_t m0) const { dma(r, voff, m0, 1); }
    void store(const Res &r, uint32_t voff, const void *data, int width) const
    {
        Request q;
        q.kind = K_STORE;
        q.a = voff;
        q.width = width;
        q.res = r;
        memcpy(q.data, data, width);
        g_emu->post(q);
    }
    void store_b128(const Res &r, uint32_t voff, u32x4 v) const
    {
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
        store(r, voff, w, 16);
    }
    void store_b32(const Res &r, uint32_t voff, uint32_t v) const { store(r, voff, &v, 4); }
    template <int K>
    void wait() const
    {
        static_assert(K >= 0 && K <= tp::kVmcntMax, "vmcnt is a 6-bit counter");
        Request q;
        q.kind = K_WAIT;
        q.a = K;
        g_emu->post(q);
    }
    void barrier() const
    {
        Request q;
        q.kind = K_BARRIER;
        g_emu->post(q);
    }
    // Device-scope accesses: the emulator's memory is one coherent store, so
    // they are the plain ones, and an 8-byte store or load is one access.
    uint32_t load_b32_device(const Res &r, uint32_t voff) const
    {
        Request q;
        q.kind = K_LOAD;
        q.a = voff;
        q.width = 4;
        q.res = r;
        g_emu->post(q);
        return g_lane->req.result;
    }
    uint64_t load_b64_device(const Res &r, uint32_t voff) const
    {
        Request q;
        q.kind = K_LOAD;
        q.a = voff;
        q.width = 8;
        q.res = r;
        g_emu->post(q);
        return g_lane->req.wide;
    }
    void store_b32_device(const Res &r, uint32_t voff, uint32_t v) const { store(r, voff, &v, 4); }
    void store_b64_device(const Res &r, uint32_t voff, uint64_t v) const { store(r, voff, &v, 8); }
    bool all_lanes(bool p) const
    {
        Request q;
        q.kind = K_ALL;
        q.a = p ? 1u : 0u;
        g_emu->post(q);
        return g_lane->req.result != 0;
    }
    void pause() const {}
};

// Status of an entry point: a tp_status from planning, 0, or these.
constexpr int kViolation = -1;       // `err` holds the first violation
constexpr int kNotInstantiated = -2; // that kernel instance is not compiled into the emulator

// Calls f(std::integral_constant<int, V>{}) for the V in the list equal to v;
// false when none is (that kernel instance is not compiled in).
template <int... V, class F>
bool pick(int v, F &&f)
{
    return ((v == V ? (f(std::integral_constant<int, V>{}), true) : false) || ...);
}

template <class Body>
int launch(const tp_plan &plan, const Options &opt, Body body, char *err, int errlen)
{
    try {
        Emulator e(opt, (uint32_t)plan.threads, (uint32_t)plan.lds_bytes, (uint32_t)plan.grid);
        g_emu = &e;
        e.run(body);
        g_emu = nullptr;
        return 0;
    } catch (const Fail &f) {
        g_emu = nullptr;
        if (err && errlen > 0)
            snprintf(err, errlen, "%s", f.what());
        return kViolation;
    }
}

}  // namespace emu
