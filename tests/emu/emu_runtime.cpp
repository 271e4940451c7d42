// Launch loop of the CPU emulation shim (test infrastructure): one thread per
// lane of a block, the grid's blocks in order, a block barrier between them.
#include "hip/hip_runtime.h"
thread_local emu_idx threadIdx, blockIdx;
thread_local dim3 blockDim, gridDim;
thread_local unsigned emu_phase;
EmuBlock *g_emu;
void emu_launch(dim3 grid, dim3 block, const std::function<void()> &body) {
    const int nt = block.x;
    EmuBarrier bb(nt);
    std::vector<EmuBarrier *> wb;
    for (int w = 0; w < nt / 64; ++w) wb.push_back(new EmuBarrier(64));
    EmuBlock e; e.nthreads = nt; e.block_bar = &bb; e.wave_bar = wb;
    e.slot.assign(nt / 64, std::vector<uint64_t>(128));
    g_emu = &e;
    std::vector<std::thread> ts;
    for (int t = 0; t < nt; ++t)
        ts.emplace_back([&, t] {
            threadIdx = {(unsigned)t, 0, 0}; blockDim = block; gridDim = grid;
            for (unsigned b = 0; b < grid.x; ++b) { blockIdx = {b, 0, 0}; body(); bb.arrive_and_wait(); }
        });
    for (auto &t : ts) t.join();
    for (auto *p : wb) delete p;
}
