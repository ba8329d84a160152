// Opt-in call log of the host API: with the environment variable JFA_LOG set
// (to anything but "0") when the library first checks it, every planner
// build and kernel entry point writes one line to stderr: its name, the
// problem, the plan's size, the status it returns and the host time it
// took (planning, validation and the asynchronous launches; not the GPU's).
#pragma once

#include <chrono>
#include <cstdint>

#include "jfa.h"

namespace jfa {

bool log_enabled();
void log_line(const char* what, const jfa_problem* p, const jfa_plan_info* info, int32_t extra,
              int32_t status, double host_us);

// Runs body (the entry point's work, returning its status) and logs the call.
template <typename F>
int32_t logged(const char* what, const jfa_problem* p, const jfa_plan_info* info, int32_t extra,
               F&& body) {
    if (!log_enabled()) return body();
    const auto t0 = std::chrono::steady_clock::now();
    const int32_t st = body();
    const double us =
        std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t0).count();
    log_line(what, p, info, extra, st, us);
    return st;
}

}  // namespace jfa
