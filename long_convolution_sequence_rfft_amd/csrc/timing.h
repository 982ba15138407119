// timing.h -- per-launch device timing for profiling (hyena_timing_* in
// include/hyena.h).  While a host thread has timing switched on, every kernel
// launch that thread makes through HY_LAUNCH is bracketed by two HIP events
// recorded on the launch stream; the label names the kernel the way the
// runtime's kernel-trace tools print it, so the two can be matched.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <sstream>
#include <string>

namespace hy {

bool timing_on();
bool log_on();
void log_msg(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
void timing_mark_begin(hipStream_t s);
void timing_mark_end(hipStream_t s, const std::string& label);

template <typename T> inline const char* type_label();
template <> inline const char* type_label<float>() { return "float"; }
template <> inline const char* type_label<uint16_t>() { return "unsigned short"; }
template <> inline const char* type_label<_Float16>() { return "_Float16"; }

inline void label_arg(std::ostringstream& o, int v) { o << v; }
inline void label_arg(std::ostringstream& o, bool v) { o << (v ? "true" : "false"); }
inline void label_arg(std::ostringstream& o, const char* v) { o << v; }

// "hy::<name><a0, a1, ...>"
template <typename... A>
std::string kernel_label(const char* name, A... args)
{
    std::ostringstream o;
    o << "hy::" << name;
    if constexpr (sizeof...(A) > 0) {
        o << '<';
        bool first = true;
        ((o << (first ? "" : ", "), label_arg(o, args), first = false), ...);
        o << '>';
    }
    return o.str();
}

}  // namespace hy

// Launch `kern` like hipLaunchKernelGGL; LABEL is an expression giving the
// label (evaluated only while timing or HYENA_LOG is on).
#define HY_LAUNCH(LABEL, kern, grid, block, lds, stream, ...)                          \
    do {                                                                              \
        const bool hy_timed_ = ::hy::timing_on();                                     \
        if (::hy::log_on()) {                                                         \
            const dim3 hy_g_ = (grid), hy_b_ = (block);                               \
            ::hy::log_msg("launch %s grid %u block %u stream %p", std::string(LABEL).c_str(), \
                          hy_g_.x, hy_b_.x, (void*)(stream));                         \
        }                                                                             \
        if (hy_timed_) ::hy::timing_mark_begin(stream);                               \
        hipLaunchKernelGGL(kern, grid, block, lds, stream, __VA_ARGS__);              \
        if (hy_timed_) ::hy::timing_mark_end(stream, LABEL);                          \
    } while (0)
